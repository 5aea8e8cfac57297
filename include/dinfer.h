/*
 * dinfer.h -- C ABI of the MI355X (gfx950) denoising-step library.
 *
 * One denoising iteration of a masked-diffusion LM over the current block:
 * vicinity KV refresh, bidirectional attention over the full cached KV, the
 * LM head with fused vocab softmax / max-probability / argmax / top-k, and the
 * parallel-decode commit (threshold, credit, top-1 fallback, optional
 * hierarchical midpoint order, iteration smoothing).
 *
 * Sources (page titles; sections):
 *   dInfer abstract, "dInfer: An Efficient Inference Framework for Diffusion
 *     Language Models": four components -- model, diffusion iteration manager,
 *     decoding strategy, KV-cache manager.  The calls below follow them:
 *     model + KV manager -> dinfer_refresh_kv / dinfer_denoise_step,
 *     decoding strategy -> dinfer_commit, iteration manager ->
 *     dinfer_advance_blocks / dinfer_run_to_completion.
 *   dInfer news article (aigc.bar), section "削减计算成本：邻近KV缓存刷新"
 *     (vicinity KV refresh), section "解码的艺术" (hierarchical, credit,
 *     smoothing), section "系统级压榨" (loop unrolling against iteration
 *     bubbles: dinfer_run_to_completion replays several steps per graph).
 *   Sangam abstract, "Sangam: Efficiently Serving Diffusion LLMs with the AR
 *     Stack": cached KV is refreshed and reused across block-sized decodes.
 *
 * Conventions for every call:
 *   - Pointers named d_* are device pointers, h_* are host pointers.
 *   - The library never allocates device memory: the caller owns the weights,
 *     token buffer and workspace, which must outlive the context.  The
 *     library borrows them.
 *   - Calls enqueue work on the context's stream and return without waiting,
 *     except dinfer_advance_blocks and dinfer_run_to_completion, which wait.
 *   - Errors are returned as dinfer_status; no exception or abort crosses the
 *     ABI.  A kernel fault surfaces as DINFER_E_HIP at the next waiting call.
 *   - Call order: step_init -> set_batch -> refresh_kv -> (denoise_step ->
 *     commit)*.  A call out of that order returns DINFER_E_STATE and changes
 *     nothing: denoise_step or step_graph before set_batch or with no
 *     refreshed request; commit without a denoise_step since the last
 *     commit, refresh_kv, advance_blocks, refill or set_batch.
 *   - A context is used from one host thread at a time.
 *
 * Layouts (row-major, no padding):
 *   Linear weights are [out][in].  tok_emb, lm_head [V][d]; wqkv [3d][d] with
 *   rows q | k | v, head-major (head h owns rows h*hd .. h*hd+hd-1 of each);
 *   w_gate_up [2F][d] with rows gate | up; w_down [d][F]; norms [d].
 *   MoE: router [E][d], exp_gate_up [E][2Fe][d], exp_down [E][d][Fe],
 *   shared_gate_up [2Fs][d], shared_down [d][Fs].
 *   Element type: float for DINFER_F32, bfloat16 for DINFER_BF16 (all
 *   weights of one model share it).
 */
#ifndef DINFER_H
#define DINFER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dinfer_ctx dinfer_ctx;

typedef enum {
  DINFER_OK = 0,
  DINFER_E_ARG = 1,          /* bad argument (null, out of range, inconsistent) */
  DINFER_E_WORKSPACE = 2,    /* workspace too small or misaligned               */
  DINFER_E_STATE = 3,        /* call out of order (e.g. denoise before refresh) */
  DINFER_E_HIP = 4,          /* a HIP runtime call failed                       */
  DINFER_E_UNSUPPORTED = 5   /* shape or option this build does not support     */
} dinfer_status;

typedef enum { DINFER_F32 = 0, DINFER_BF16 = 1 } dinfer_dtype;

/* Model: a bidirectional (non-causal) pre-norm transformer with RoPE,
 * RMSNorm and SwiGLU; n_experts == 0 selects the dense FFN.  Supported:
 * head_dim 64 or 128; MoE with n_experts <= 64, top_k <= 8 and d_model a
 * multiple of 512 (bf16) / 256 (f32); others give DINFER_E_ARG at init. */
typedef struct {
  int32_t n_layers, d_model, n_heads, head_dim, ffn_dim, vocab, mask_id;
  int32_t n_experts, top_k, expert_ffn, shared_ffn;
  float rope_theta, rms_eps;
  int32_t dtype;             /* dinfer_dtype */
} dinfer_model_cfg;

/* Decoding strategy (dInfer news article, section "解码的艺术"). */
typedef struct {
  int32_t block_len;         /* B: positions per block, 1..64                    */
  int32_t vicinity_w;        /* w: window = [max(0,bs-w), min(L,be+w))           */
  float tau;                 /* confidence threshold, inclusive                  */
  float credit_weight;       /* lambda; 0 = plain threshold decoding             */
  float credit_decay;        /* gamma                                            */
  float credit_kappa;        /* credit gate, inclusive                           */
  float smooth_alpha;        /* 0 = no iteration smoothing                       */
  int32_t smooth_topk;       /* must be 8                                        */
  int32_t hierarchical;      /* 1 = only run midpoints are candidates            */
  int32_t graph_unroll;      /* steps per captured graph in run_to_completion;
                                0 = launch eagerly                               */
  int32_t eos_id;            /* -1 = none.  Else the end-of-sequence token (early
                                stop, dInfer news article, section "系统级压榨"):
                                once a request holds it at a response position
                                p, every still-masked response position after p
                                takes it, and a request left with no masked
                                response position is complete (its remaining
                                blocks get neither refresh nor steps).  Must be
                                in [0, vocab) and differ from mask_id.          */
} dinfer_decode_cfg;

/* Device pointers to the weights (borrowed).  Per-layer entries are host
 * arrays of n_layers device pointers; unused families may be NULL.
 * Projection weights -- lm_head, wqkv, wo, w_gate_up, w_down, exp_gate_up,
 * exp_down, shared_gate_up, shared_down -- are Linear [out][in] matrices
 * (experts: [E][out][in]) in the packed layout of dinfer_pack_linear; the
 * others (tok_emb [V][d], norms [d], router [E][d]) are plain row-major. */
typedef struct {
  const void* tok_emb;
  const void* final_norm;
  const void* lm_head;
  const void* const* attn_norm;
  const void* const* wqkv;
  const void* const* wo;
  const void* const* ffn_norm;
  const void* const* w_gate_up;
  const void* const* w_down;
  const void* const* router;
  const void* const* exp_gate_up;
  const void* const* exp_down;
  const void* const* shared_gate_up;
  const void* const* shared_down;
} dinfer_weights;

typedef struct {
  int64_t steps;             /* denoise+commit steps launched                    */
  int64_t refreshes;         /* per-request block-start refreshes                */
  int64_t committed;         /* tokens committed over all requests               */
  double wall_ms;            /* wall time of the call                            */
  double refresh_ms;         /* part of wall_ms spent in refreshes (event-timed) */
} dinfer_run_stats;

/* Device pointers into the context's state, for inspection and tests.  All
 * buffers are indexed by request r < batch and block offset j < block_len:
 * row index = r * block_len + j. */
typedef struct {
  int32_t batch, block_len, vocab, topk;
  float* logits;             /* [batch*B][V] fp32 logits of the block rows (before
                                planting bias and MASK exclusion), written by
                                denoise_step only while dinfer_keep_logits is
                                on (the statistics never read them)             */
  int32_t* argmax;           /* [batch*B]                                        */
  float* conf;               /* [batch*B] max softmax probability                */
  float* lse;                /* [batch*B] log-sum-exp                            */
  int32_t* topk_id;          /* [batch*B][8]                                     */
  float* topk_p;             /* [batch*B][8] softmax probabilities               */
  float* credit;             /* [batch*B]                                        */
  int32_t* tracked;          /* [batch*B] argmax tracked by credit (-1 = none)   */
  int32_t* smooth_id;        /* [batch*B][8] smoothing ids                       */
  float* smooth_p;           /* [batch*B][8] renormalised smoothing probs        */
  uint8_t* smooth_valid;     /* [batch*B]                                        */
  uint8_t* commit_mask;      /* [batch*B] 1 = committed by the last commit       */
  int32_t* block_done;       /* [batch] 1 once the current block has no MASK,
                                2 once the whole response has none (EOS)        */
  int32_t* step_count;       /* [batch] steps taken in the current block         */
  int32_t* commit_count;     /* [batch] tokens committed in total                */
  void* kv_k;                /* [n_layers][max_batch][H][kv_len][hd] K, RoPE'd  */
  void* kv_v;                /* [n_layers][max_batch][H][kv_len/32][hd][32] V in
                                transposed tiles of 32 positions                 */
  /* MoE only (else 0 / NULL): routing of the last layer whose FFN the last
   * pass ran (a step runs every layer; a refresh stops before the last
   * layer's FFN), one row per pass row in pass order (request by request,
   * positions ascending: a step's window, or every position of each refreshed
   * request).  Row m holds its top_k experts (router logit descending, lower
   * id first on ties) and their gates renormalised over the selection. */
  int32_t moe_top_k;
  int32_t* moe_sel;          /* [rows][moe_top_k]                                */
  float* moe_gate;           /* [rows][moe_top_k]                                */
  int32_t moe_experts;       /* E                                                */
  float* moe_logits;         /* [rows][E] router logits incl. the block's bias   */
  /* After a step: [rows][d] fp32 normalised FFN input of the last layer, rows
   * in pass order (after a refresh it holds other intermediate values).  For
   * a dense bf16 model whose step row capacity m = max_batch * min(max_len,
   * block_len + 2 * vicinity_w) exceeds 128 it holds the same values as two
   * bf16 planes, hi = bf16(a) [m][d] then lo = bf16(a - hi) [m][d], the form
   * its projections read. */
  float* ffn_in;
  int32_t kv_len;            /* cache positions per head row: max_len rounded up
                                to a multiple of 64 (padding holds zeros)        */
  /* Decode accounting of each request since set_batch (or its refill):
   * [batch][decode_stat_words] int32 -- [0] commits through the threshold
   * gate, [1] through the credit gate alone, [2] through the fallback, [3]
   * steps that found the request's block already done (graph replays past a
   * block's end), [4 + k] steps that committed k tokens, k = 0..64.
   * Statistics only: nothing reads them back. */
  int32_t* decode_stats;
  int32_t decode_stat_words;
} dinfer_step_view;

/* Bytes of workspace dinfer_step_init needs for these shapes (0 on bad args). */
size_t dinfer_workspace_bytes(const dinfer_model_cfg* model, const dinfer_decode_cfg* dec,
                              int32_t max_batch, int32_t max_len);

/* Validate the configuration, carve the caller's workspace (256-byte aligned,
 * at least dinfer_workspace_bytes), build the RoPE tables and bind the
 * stream (a hipStream_t; NULL = the default stream).  *out receives the
 * context.  Model and KV-cache manager set-up (dInfer abstract). */
dinfer_status dinfer_step_init(const dinfer_model_cfg* model, const dinfer_decode_cfg* dec,
                               const dinfer_weights* weights, int32_t max_batch, int32_t max_len,
                               void* d_workspace, size_t ws_bytes, void* stream,
                               dinfer_ctx** out);

/* Bind a batch of requests.  d_tokens [batch][max_len] int32 holds each
 * request's prompt then MASK positions and is updated in place by commits.
 * h_prompt_len / h_gen_len [batch]: gen_len must be a multiple of block_len
 * and prompt_len + gen_len <= max_len.  d_plant_id [batch][max_len] int32
 * (-1 = no planting) and d_plant_bias [batch] float: the planted target of a
 * position gets +bias on its raw logit before the vocab statistics.
 * d_router_bias (MoE only, else NULL; a dense model rejects it with
 * DINFER_E_ARG): [batch][n_layers][nb][E] float with nb = max over the batch
 * of gen_len/B; entry [r][l][k] is added to the router logits of layer l for
 * every row of request r while r works on block k (refresh and steps).  The
 * array stays owned by the caller and must live until the next set_batch.
 * Every request starts at block 0; call dinfer_refresh_kv next. */
dinfer_status dinfer_set_batch(dinfer_ctx* ctx, int32_t batch, int32_t* d_tokens,
                               const int32_t* h_prompt_len, const int32_t* h_gen_len,
                               const int32_t* d_plant_id, const float* d_plant_bias,
                               const float* d_router_bias);

/* KV-cache manager, full refresh (Sangam abstract: cached KV is refreshed and
 * reused across the decodes in between).  For every selected request
 * (h_req_mask[r] != 0; NULL = every request with an unfinished block):
 * recompute K and V of all its positions from hard embeddings, and start its
 * current block (credit, tracked ids and smoothing state cleared). */
dinfer_status dinfer_refresh_kv(dinfer_ctx* ctx, const uint8_t* h_req_mask);

/* Model + vicinity refresh (dInfer news article, section
 * "削减计算成本：邻近KV缓存刷新"): for every active request, the window rows
 * run through all layers; per layer their fresh K,V are written into the
 * cache before they attend over all cached positions (no causal mask).  The
 * block rows then go through the final norm, the LM head and the vocab
 * statistics (planting bias, MASK excluded, argmax lowest id on ties,
 * max-probability, log-sum-exp, top-8).  Results: dinfer_get_step_view. */
dinfer_status dinfer_denoise_step(dinfer_ctx* ctx);

/* Decoding strategy (dInfer news article, section "解码的艺术"): per active
 * request, credit update of every still-masked block position
 * c <- (argmax == tracked ? gamma*c : 0) + lambda*p (fp32, two roundings),
 * candidates (all masked positions, or the midpoints of maximal masked runs
 * when hierarchical), commit every candidate with p >= tau or c >= kappa,
 * else the single candidate of highest p (lowest position on ties); write
 * the committed ids into d_tokens; keep each still-masked position's top-8
 * (renormalised) for the next step's soft embedding; set block_done when the
 * block holds no MASK. */
dinfer_status dinfer_commit(dinfer_ctx* ctx);

/* Iteration manager, block bookkeeping: waits for the stream, then for every
 * request whose block is done moves to its next block (or marks it
 * finished).  h_needs_refresh[r] (may be NULL) is set to 1 for unfinished
 * requests whose current block has not been refreshed (moved to a new block,
 * or a refilled slot): they must be refreshed before the next step.
 * *h_unfinished (may be NULL) receives the number of unfinished requests. */
dinfer_status dinfer_advance_blocks(dinfer_ctx* ctx, uint8_t* h_needs_refresh,
                                    int32_t* h_unfinished);

/* Iteration manager, continuous batching (serving-characterisation page
 * "服务掩码扩散大语言模型：来自真实硬件的特征分析与设计原则", section "Design
 * Principles for Future Systems": step-level parallelism, request admission
 * and eviction between shared forward passes): restart the finished slot
 * `slot` with a new request.  Before the call the caller writes the new
 * request into the slot's rows of the arrays given to dinfer_set_batch:
 * tokens[slot] (prompt ids, then mask_id over the response), plant
 * ids[slot] and plant bias[slot], and with an MoE router bias its
 * [slot] entries.  The slot restarts at block 0, waits for the next
 * dinfer_refresh_kv that selects it (dinfer_advance_blocks reports it in
 * h_needs_refresh until then), and its step and commit counters restart at
 * 0 (a reset enqueued on the context's stream).  DINFER_E_STATE if the slot
 * has not finished; DINFER_E_ARG for lengths dinfer_set_batch would reject
 * or, with a router bias, more blocks than dinfer_set_batch sized it for. */
dinfer_status dinfer_refill(dinfer_ctx* ctx, int32_t slot, int32_t prompt_len, int32_t gen_len);

/* h_finished[r] = 1 for every request r of the batch that has finished
 * (host bookkeeping of dinfer_advance_blocks; no wait). */
dinfer_status dinfer_finished(const dinfer_ctx* ctx, uint8_t* h_finished);

/* Per-slot token cost of the next scheduling round (host bookkeeping, no
 * wait): h_decode_rows[r] = rows of request r's next denoising step (its
 * block with the +-w window, clipped to the request) if r is refreshed and
 * unfinished, else 0; h_refresh_rows[r] = prompt + response length (the rows
 * of a whole refresh) if r is unfinished and waits for a refresh, else 0.
 * Both arrays hold `batch` entries.  DINFER_E_STATE before dinfer_set_batch. */
dinfer_status dinfer_pending_rows(const dinfer_ctx* ctx, int32_t* h_decode_rows,
                                  int32_t* h_refresh_rows);

/* Deficit token-budget admission of whole KV refreshes ("Sangam: Efficiently
 * Serving Diffusion LLMs with the AR Stack", abstract: in-flight decodes are
 * admitted first, a whole refresh -- which bidirectional attention does not
 * let one split -- only when the token budget accumulated so far covers it,
 * unused budget carries over).  A host-only object; no GPU work, no context.
 *
 * One round per forward pass: the counter gains token_budget, loses the rows
 * of every decode of the round, and then admits waiting slots first come
 * first served (slots that start to wait in the same round queue in slot
 * order) while it covers the head's rows; the head of the queue blocks the
 * slots behind it.  In a round with no decode the head is admitted even if
 * the counter does not cover it (the counter goes negative).  When no slot is
 * left waiting at the end of a round the counter returns to 0, so budget is
 * carried only while a refresh waits.
 *
 * dinfer_sched_create: token_budget in [0, 2^62] rows per round, n_slots >= 1;
 * *out receives the object (NULL on error).  dinfer_sched_destroy frees it
 * (NULL is a no-op).  dinfer_sched_round: h_decode_rows[r] > 0 for a slot
 * decoding in this round, h_refresh_rows[r] > 0 for a slot waiting for a
 * refresh (n_slots entries each, both >= 0, at most one of the two > 0 per
 * slot, else DINFER_E_ARG and the state is unchanged); a queued slot whose
 * refresh_rows becomes 0 leaves the queue.  h_admit[r] = 1 for the slots
 * admitted in this round; *h_deficit (may be NULL) receives the counter after
 * the round.  The caller refreshes the admitted slots before the round's
 * step.  Not thread-safe per object. */
typedef struct dinfer_sched dinfer_sched;
dinfer_status dinfer_sched_create(int64_t token_budget, int32_t n_slots, dinfer_sched** out);
void dinfer_sched_destroy(dinfer_sched* sched);
dinfer_status dinfer_sched_round(dinfer_sched* sched, const int32_t* h_decode_rows,
                                 const int32_t* h_refresh_rows, uint8_t* h_admit,
                                 int64_t* h_deficit);

/* Iteration manager: run every request of the batch to completion --
 * refresh at each block start, then denoise+commit steps replayed
 * graph_unroll at a time from a captured HIP graph (one host wait per
 * replay), until every block of every request is committed or max_steps
 * steps ran (DINFER_E_STATE then).  h_stats may be NULL. */
dinfer_status dinfer_run_to_completion(dinfer_ctx* ctx, int32_t max_steps,
                                       dinfer_run_stats* h_stats);

/* TIDE-style interval expert placement ("TIDE: Efficient and Lossless MoE
 * Diffusion LLM Inference with I/O-aware Expert Offload", abstract: expert
 * activations are stable over the steps of a block, so the placement of
 * experts is refreshed at intervals, moving only what changes, without loss).
 *
 * dinfer_expert_offload switches an MoE context to an expert cache: every
 * expert of every layer lives in a host store (h_exp_gate_up[l],
 * h_exp_down[l]: per layer the packed [E][2Fe][d] and [E][d][Fe] matrices of
 * dinfer_pack_linear, in pinned host memory from hipHostMalloc, borrowed),
 * and `slots` experts per layer are also held in HBM, in d_slots (caller
 * device memory, 256-byte aligned, at least n_layers * slots *
 * dinfer_expert_slot_bytes bytes, borrowed).  The grouped expert projection
 * reads a resident expert from its slot and any other expert directly from
 * the host store, so every result is bit-identical to the all-in-HBM run;
 * only the time changes.  The experts given to dinfer_step_init are not used
 * afterwards (they may be NULL there, both arrays, if this call follows
 * before the first refresh).  Initially experts 0..slots-1 are resident.
 * Placement: per layer, the `slots` experts with the most row assignments
 * since the last block-start placement (ties: the resident one, then the
 * lower id) are copied into the slots of the experts they replace (on the
 * context's stream, in order with the kernels).  dinfer_run_to_completion
 * places after every block-start refresh (ranking by that refresh's routing
 * and the steps before it, then restarting the counts) and, with
 * interval > 0, every `interval` steps inside a block (rounded up to whole
 * graph replays; ranking by everything the block has routed so far, counts
 * kept); dinfer_expert_place does a block-start placement on demand (waits
 * for the stream).  DINFER_E_STATE if called twice; DINFER_E_WORKSPACE for a
 * bad slot buffer; DINFER_E_ARG for a dense model or memory that is not
 * pinned host memory. */
typedef struct {
  int64_t expert_hits;       /* (layer, pass, expert) with rows, expert resident */
  int64_t expert_misses;     /* ... expert read from the host store              */
  int64_t row_hits;          /* row assignments to resident experts              */
  int64_t row_misses;        /* row assignments to host-store experts            */
  int64_t bytes_placed;      /* host -> HBM copies of placements                 */
  int64_t bytes_host_read;   /* expert_misses x one expert's weight bytes: what
                                the kernels read from host memory at least       */
  int64_t placements;
  int32_t slots, interval;
} dinfer_expert_cache_stats;
size_t dinfer_expert_slot_bytes(const dinfer_model_cfg* model);
dinfer_status dinfer_expert_offload(dinfer_ctx* ctx, const void* const* h_exp_gate_up,
                                    const void* const* h_exp_down, int32_t slots,
                                    int32_t interval, void* d_slots, size_t slots_bytes);
dinfer_status dinfer_expert_place(dinfer_ctx* ctx);
/* Counters since dinfer_expert_offload (or the last reset); waits for the
 * stream.  reset != 0 clears them after reading. */
dinfer_status dinfer_expert_cache_report(dinfer_ctx* ctx, dinfer_expert_cache_stats* out,
                                         int32_t reset);

/* Activation precision of the projections (bf16 weights; default 0, 0):
 * bit i of a mask set means projection i -- 0 QKV, 1 O, 2 gate|up, 3 down
 * (for an MoE model: the shared expert's gate|up and down) -- takes its fp32
 * activations into the bf16 MFMA as bf16(a) alone, one MFMA per weight
 * fragment; clear means as hi = bf16(a) plus lo = bf16(a - hi), two MFMAs, so
 * that only the weights' rounding remains.  Bit 4 does the same for the
 * attention's probabilities in its P V product (the queries keep both
 * halves).  step_mask applies to denoise_step, refresh_mask to refresh_kv.
 * DINFER_E_ARG for bits above 4; DINFER_E_UNSUPPORTED with fp32 weights and
 * a nonzero mask. */
dinfer_status dinfer_set_activation_precision(dinfer_ctx* ctx, uint32_t step_mask,
                                              uint32_t refresh_mask);

/* Inspection switch (default off): while on, denoise_step also stores the
 * block rows' fp32 logits into the step view's logits buffer.  The vocab
 * statistics are computed in the LM head's epilogue either way (per row and
 * column tile: planting bias, MASK exclusion, max, sum of exp, top-8; then a
 * merge per row), so the switch changes no result, only the extra store.
 * Takes effect at the next denoise_step (a captured step graph is dropped
 * and captured again). */
dinfer_status dinfer_keep_logits(dinfer_ctx* ctx, int32_t on);

/* Fill *out with device pointers into the context's state. */
dinfer_status dinfer_get_step_view(const dinfer_ctx* ctx, dinfer_step_view* out);

/* Launch n_steps denoise+commit steps without waiting and without block
 * bookkeeping: the captured graph of graph_unroll steps (captured on first
 * use) is replayed n_steps / graph_unroll times (n_steps must be a multiple
 * of graph_unroll, graph_unroll > 0).  Requests whose block completes
 * mid-way stop committing (their window is still recomputed).  The loop
 * unrolling of the dInfer news article, section "系统级压榨". */
dinfer_status dinfer_step_graph(dinfer_ctx* ctx, int32_t n_steps);

/* Weight packing (a storage format of this library, not of the method):
 * copies d_W, a stack of n_mats row-major matrices [n_mats][rows][K] of the
 * given dtype (one Linear [out][in] weight: n_mats = 1; MoE experts [E][N][K]:
 * n_mats = E), into d_packed (same byte size, no overlap) in the layout every
 * projection kernel reads; each matrix is packed on its own.  A block is the
 * 1 KB MFMA operand of 16 rows (a group) x one run of 32 (bf16) / 16 (f32)
 * columns: its 16-byte slot 16*q + c holds row c of the group, columns
 * q*VEC .. q*VEC+VEC-1 of the run (VEC = 8 bf16 / 4 f32).  Blocks are
 * stored run-major: block (group g, run s) is at index s*(rows/16) + g, with
 * KS = K/32 (bf16) or K/16 (f32) runs.  A wave's weight load is then one
 * contiguous kilobyte, a workgroup's column tile one contiguous piece per
 * run, and the workgroups of one K split read neighbouring pieces as they
 * advance together (a narrow address window sweeping through the matrix).
 * rows % 16 == 0; K a multiple of 32 (bf16) / 16 (f32); n_mats <= 65535.
 * Enqueued on stream. */
dinfer_status dinfer_pack_linear(const void* d_W, void* d_packed, int32_t n_mats, int32_t rows,
                                 int32_t K, int32_t dtype, void* stream);

/* Standalone projection, the Linear layer every step runs:
 * out[s][m][n] = sum over the s-th K slice of A[m][k] * W[n][k], with A an fp32
 * [M][K] row-major device array (activations are fp32 throughout the step)
 * and W [N][K] in the model dtype, packed by dinfer_pack_linear; out fp32
 * [splits][M][N].  The
 * product A W^T is the sum of the splits (taken in split order by the
 * library's own consumers).  With bf16 weights each activation enters the
 * MFMA as hi = bf16(a) plus lo = bf16(a - hi), so only the weights' rounding
 * remains.  *h_splits (may be NULL) receives the split count; out must hold
 * dinfer_linear_out_elems(M, N, K, dtype) floats.  Requires N % 128 == 0 and
 * K % 128 == 0 (bf16) / K % 64 == 0 (f32).  Same kernels and launch plan as
 * the step for the same M. */
size_t dinfer_linear_out_elems(int32_t M, int32_t N, int32_t K, int32_t dtype);
dinfer_status dinfer_linear(const float* d_A, const void* d_W, float* d_out, int32_t M, int32_t N,
                            int32_t K, int32_t dtype, int32_t* h_splits, void* stream);

/* Standalone vocab statistics over materialised fp32 logits d_logits
 * [rows][vocab] -- the statistics dinfer_denoise_step computes in its LM
 * head's epilogue without storing logits, here as a pass of its own:
 * d_plant_id [rows] (-1 none) and d_plant_bias [rows] add the planting bias;
 * mask_id is excluded (-1 = none).  Outputs: d_argmax [rows], d_conf [rows],
 * d_lse [rows], d_topk_id [rows][8], d_topk_p [rows][8].  d_scratch must hold
 * dinfer_vocab_stats_scratch_bytes(rows, vocab) bytes.  Enqueued on stream. */
size_t dinfer_vocab_stats_scratch_bytes(int32_t rows, int32_t vocab);
dinfer_status dinfer_vocab_stats(const float* d_logits, int32_t rows, int32_t vocab,
                                 const int32_t* d_plant_id, const float* d_plant_bias,
                                 int32_t mask_id, int32_t* d_argmax, float* d_conf,
                                 float* d_lse, int32_t* d_topk_id, float* d_topk_p,
                                 void* d_scratch, size_t scratch_bytes, void* stream);

/* dinfer_vocab_stats without a scratch argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels, with the split partials
 * in a fixed 2 MiB array of device memory that the library holds on each GPU
 * it runs on until the process ends.  Makes no allocation.  Returns
 * DINFER_E_UNSUPPORTED when rows x vocab splits need more than that
 * (dinfer_vocab_stats_scratch_bytes(rows, vocab) > 2 MiB: about 29000 rows
 * at vocab 126464).  Calls on one GPU share its array: calls that may overlap
 * on one GPU (different streams, no ordering between them) race and must not
 * be issued; calls ordered on one stream are safe.  Other arguments and
 * errors as dinfer_vocab_stats. */
dinfer_status dinfer_vocab_stats_noalloc(const float* d_logits, int32_t rows, int32_t vocab,
                                         const int32_t* d_plant_id, const float* d_plant_bias,
                                         int32_t mask_id, int32_t* d_argmax, float* d_conf,
                                         float* d_lse, int32_t* d_topk_id, float* d_topk_p,
                                         void* stream);

/* Human-readable name of a status; the last error message of the calling
 * thread is appended by dinfer_last_error. */
const char* dinfer_status_str(dinfer_status s);
const char* dinfer_last_error(void);

/* Release the context (host memory, streams and graphs it created).  The
 * caller's device buffers are untouched. */
void dinfer_destroy(dinfer_ctx* ctx);

#ifdef __cplusplus
}
#endif

#endif /* DINFER_H */
