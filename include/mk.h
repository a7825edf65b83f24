/* mk.h -- C ABI of the persistent-megakernel decode library (libmk.so), MI355X / gfx950.
 *
 * One transformer decode step of a Llama-family model (RMSNorm, QKV projection,
 * RoPE, KV-cache write, split-KV decode attention, output projection, SwiGLU
 * FFN, final RMSNorm, LM head, argmax) runs as ONE resident grid: one
 * workgroup per compute unit executes a static queue of tile instructions that
 * the host planned once, and tile-level event counters in device memory replace
 * kernel boundaries.  The design follows the pages this library was written
 * from: the MegaRTP article (tahou.com), sections 3-4 (host-generated
 * instruction queues [num_CUs, max_len, 32] int32 with NoOp padding, event
 * counters with thresholds, an operand pointer table [num_ops, 16] u64, worker
 * roles, recycled shared-memory pages); the CMU 15-779 lecture 7 notes
 * (semidirectx.com), sections 4-6 (worker loop: prefetch weights before waiting
 * on counters; per-layer task partition; MPK task graph); the MPK internals
 * notes (dpshk.com) for gcd/lcm event partitioning and linearization.
 *
 * Conventions shared by every call:
 *  - No exception crosses the ABI.  Every call returns an mk_status; on failure
 *    mk_last_error() gives a thread-local message for the last failing call.
 *  - "host" pointers are CPU memory read during the call only; "device"
 *    pointers are HIP device memory that must stay valid until the stream work
 *    that uses them has completed.  The caller owns weights, KV cache, token
 *    ids and streams; a plan owns its queues, counters, workspace and outputs.
 *  - One in-flight run per plan (counters and workspace belong to the plan);
 *    distinct plans are independent.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_ABI_VERSION 2

typedef enum {
  MK_OK = 0,
  MK_E_INVALID = -1,     /* bad pointer, size or state of an argument */
  MK_E_UNSUPPORTED = -2, /* a shape or option outside what the library supports */
  MK_E_NOMEM = -3,       /* host or device allocation failed */
  MK_E_HIP = -4,         /* a HIP runtime call failed (message has hipGetErrorString) */
  MK_E_TIMEOUT = -5,     /* a device-side wait exceeded its bound (watchdog record filled) */
  MK_E_STATE = -6        /* the call does not apply to this plan (e.g. running a graph-only plan) */
} mk_status;

typedef struct mk_plan mk_plan; /* opaque */

/* Thread-local text for the last failing call on this thread ("" if none). */
const char* mk_last_error(void);
int mk_abi_version(void);

/* ---------------------------------------------------------------------------
 * Model description.  Plain data, copied by mk_plan_build.
 * arch: MK_ARCH_LLAMA (RMSNorm, GQA attention, SwiGLU) or MK_ARCH_QWEN3 (adds a
 * per-head RMSNorm of q and k before RoPE, weights q_norm/k_norm, same eps).
 * weight_dtype: MK_BF16 (row-major [out, in], PyTorch Linear layout).
 * max_kv_len: rows per sequence in the KV cache (capacity); kv_len[b] + 1 <= it.
 * RoPE is rotate-half with angle pos * rope_theta^(-2i/head_dim).
 *
 * MK_ARCH_GLM_PREATTN: the GLM-style path before sparse MLA (MegaRTP article,
 * sections 1 and 4) for M = batch token rows (1..16), rows_per_seq rows per
 * request (row m belongs to request m / rows_per_seq, kv_len[m] is its cache
 * position): h = x + r, r_out = bf16(h); y = RMSNorm(h) * attn_norm; y is
 * quantized to OCP E4M3 per (row, 128 columns) with scale max(amax, 1e-4) / 448;
 * three independent branches: QKV-A (y8 -> q_lora + kv_lora + rope_dim), head
 * gate (y -> n_gate, fp32 output) and indexer-K (y8 -> idx_head_dim, bf16 into
 * the indexer cache); the q columns are RMSNorm'd (q_a_norm) and requantized,
 * then QKV-B (-> n_q_heads x head_dim, rotate-half RoPE on each head's last
 * rope_dim dims, bf16 output) and indexer-Q (-> n_idx_heads x idx_head_dim,
 * bf16 output); the KV row [RMSNorm(kv) * kv_a_norm | RoPE(k_rope)] (bf16) is
 * written at the row's position.  weight_dtype MK_FP8_E4M3_B128: linear
 * weights are E4M3 codes [out, in] with fp32 scales [ceil(out/128)][in/128].
 * Fields used: hidden, n_q_heads, head_dim, max_kv_len, rms_eps, rope_theta
 * and the GLM fields below (n_layers must be 1; the Llama-only fields are ignored).
 * Supported: hidden (<= 8192) and q_lora (<= 3072) multiples of 128, kv_lora
 * (<= 1024) a multiple of 8 with kv_lora + rope_dim a multiple of 8, head_dim -
 * rope_dim and rope_dim positive multiples of 16 with each head's rope dims
 * inside one 128-row scale block, n_gate, idx_head_dim and n_idx_heads *
 * idx_head_dim multiples of 16 (64, 128, 4096 for the GLM shape).  The head
 * gate is planned as K-split tiles (4 blocks of 128 columns each) and a reduce
 * op that adds their partials in split order.
 * ------------------------------------------------------------------------- */
enum { MK_ARCH_LLAMA = 1, MK_ARCH_QWEN3 = 2, MK_ARCH_GLM_PREATTN = 3 };
enum { MK_BF16 = 0, MK_FP8_E4M3_B128 = 1 };

typedef struct {
  uint32_t abi_version; /* MK_ABI_VERSION */
  uint32_t struct_size; /* sizeof(mk_model_desc) */
  int32_t arch;
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  int32_t tied_lm_head; /* 1: the LM head is the embedding matrix */
  int32_t qk_norm;      /* 1 for MK_ARCH_QWEN3 */
  int32_t weight_dtype; /* MK_BF16 */
  int32_t max_kv_len;   /* KV-cache capacity per sequence (rows) */
  float rms_eps, rope_theta;
  /* MK_ARCH_GLM_PREATTN only (0 otherwise) */
  int32_t q_lora, kv_lora, rope_dim, n_idx_heads, idx_head_dim, n_gate, rows_per_seq;
} mk_model_desc;

/* Planning options; pass NULL (or 0 in a field) for the defaults.
 * num_cus: workgroups of the persistent grid = queues (default: the device's CU
 *   count; the plan can be built without a GPU when it is given).
 * gemv_rows: weight rows per QKV / O / LM-head tile (default 32768 / hidden,
 *   clamped to [4, 16]); gateup_outs: FFN outputs per gate/up tile (default
 *   gemv_rows / 2); down_rows: rows per down tile (default 32768 / ffn at
 *   batch 1, 65536 / ffn above, clamped to [1, 16]); lm_rows: LM-head rows per
 *   tile (default gemv_rows);
 * attn_splits: KV splits per (sequence, kv head) (default from the longest
 *   sequence: ceil((kv+1)/64) clamped to [1, 32], lowered to
 *   ceil(2 num_cus / (batch n_kv_heads)) when that is smaller; while the
 *   batch n_kv_heads S tasks still fit on num_cus at one each, lowered until
 *   they fit on 7/8 of them; then raised until one split's K and V rows fit in
 *   64 KiB, or in the page ring less 64 KiB while the tasks fit on num_cus at
 *   one each; batched head_dim-64 tasks stream their rows through the ring and
 *   skip the raise);
 * timeout_ms: bound of every device-side wait (default 200);
 * dma_pages: 16 KiB pages each of the two weight-loader waves may leave in
 *   flight behind the one it is issuing (1 to 3, default 1): the event polls and
 *   activation reads that carry the dependency chain queue behind the page DMA,
 *   and more bytes in flight lengthen those queues without raising the stream
 *   rate, so a shallow backlog is the default.  Does not change the plan's
 *   schedule metadata.
 * lw_streams: streams of mk_run_layerwise (0 or 1: every launch on the caller's
 *   stream; 2 or 3: independent branches of the op graph -- the GLM path's QKV-A,
 *   head gate and indexer-K after A0, QKV-B and indexer-Q after the q-path norm --
 *   on streams of their own, forked from and joined back into the caller's stream
 *   with events, also under stream capture; a chain, like the Llama-family
 *   graph, stays on one stream).  Eager GLM steps are slower with branches (the
 *   event hand-offs cost more than the branches overlap); captured in a graph
 *   they time the same as one stream.
 * pairing (Llama family): 0 (default) derives events with the gcd/lcm rules
 *   below; 1 plans with the pairing strategies of mk_pair_plan instead (MegaRTP
 *   article, section 4, "TaskGraph"): QKV tiles cover their kv head's rows,
 *   attention splits are partials reduced by combine, every other input is read
 *   whole, and the residual inputs stay explicit, so O waits on combine and on
 *   the previous layer's down, and down on gate/up and on O (two waits per
 *   instruction).  Tasks op by op in grid order.
 * attn_order (Llama family): 1 places attention tasks longest first (CMU
 *   15-779 lecture 7 notes, section 6.4, variable-length tasks): within each
 *   run of consecutive attention tasks that wait on the same events, tasks are
 *   taken in decreasing KV rows (ties in task order), each on the free position
 *   of the run whose queue holds the least attention rows of that layer so far
 *   (ties: lowest position); it moves tasks only within such runs, so the events
 *   and their thresholds are unchanged.  -1 leaves them in plan order.  0
 *   (default): longest first at batch 2..16 (sequences of different lengths),
 *   plan order at batch 1. */
typedef struct {
  int32_t num_cus, gemv_rows, gateup_outs, down_rows, lm_rows, attn_splits;
  int32_t timeout_ms;
  int32_t dma_pages;
  int32_t lw_streams;
  int32_t pairing;
  int32_t attn_order;
  int32_t reserved;
} mk_plan_opts;

/* Build the static tile plan of one decode step (host-only arithmetic; uploads
 * nothing until the first run).  Defined by: MegaRTP article, section 4
 * ("TaskGraph": tiles to counter events; "KernelPlan": round-robin queues of
 * 32-word instructions padded with NoOps; the operand pointer table); MPK
 * internals notes, "fine-grained pipeline" (per-dimension gcd of the producer
 * and consumer partitions), "handling fork producer" / "handling join
 * consumer" (lcm normalization) and "building the SM-level DAG"
 * (linearization); CMU 15-779 lecture 7 notes, section 6 (per-layer task
 * partition of the decode step).  kv_len: host int32[batch], prior rows per
 * sequence; the step writes row kv_len[b] and attends rows 0..kv_len[b].  The
 * planner cuts every operator into tiles, derives events by gcd partition of
 * each producer/consumer edge (lcm-normalized at forks and joins), drops
 * residual edges implied transitively, linearizes tasks so each event's
 * successors are contiguous, and places task t in queue t % num_cus at slot
 * t / num_cus.  Deterministic: equal inputs give bit-identical plans.
 * Errors: MK_E_INVALID (null/size/abi mismatch), MK_E_UNSUPPORTED (head_dim not
 * 64 or 128, hidden or ffn not a multiple of 8 or above 12288, more than 4 query
 * heads per kv head, kv_len[b] + 1 > max_kv_len, batch outside 1..16, batch-1
 * GEMV tiles with more rows than their K allows (16 up to K 2048, 8 up to 4096,
 * 4 beyond), tiles that do not fit the LDS page ring: 144 KiB at batch 1, 128
 * KiB at batch 2..16; batched head_dim-64 attention tasks stream their K/V rows
 * through the ring in chunks of 32 positions and may be longer).  Batch 1 runs fp32 vector GEMV tiles; batch 2..16 runs the
 * same tiles on the matrix cores (16 weight rows x 16 sequences per MFMA block,
 * activations entered as bf16 high and low parts). */
mk_status mk_plan_build(const mk_model_desc* desc, int32_t batch, const int32_t* kv_len,
                        const mk_plan_opts* opts, mk_plan** out);

/* Plan an arbitrary operator graph with the same rules (no payloads; the result
 * can be exported but not run: mk_run returns MK_E_STATE).  Defined by the MPK
 * internals notes' worked examples (fork producer, join consumer, gcd table).  ops[i].grid holds
 * up to three axis extents; edges must go from a lower to a higher op index;
 * out_map / in_map give, per grid axis, the tensor dimension (0..3) it
 * partitions or -1; when has_extent is set, extent/ptile/ctile (elements) let
 * the planner reject gcd slices that do not cut the tensor at the same places
 * on both sides (ragged tiles). */
typedef struct {
  int32_t opcode, spec, layer;
  int32_t grid[3];
} mk_graph_op;
typedef struct {
  int32_t prod, cons;
  int32_t out_map[3], in_map[3];
  int32_t has_extent;
  int32_t extent[4], ptile[4], ctile[4];
} mk_graph_edge;
mk_status mk_graph_plan(const mk_graph_op* ops, int32_t n_ops, const mk_graph_edge* edges, int32_t n_edges,
                        int32_t num_cus, mk_plan** out);

/* Plan an operator graph under the pairing strategies (MegaRTP article,
 * section 4, "TaskGraph" and "KernelPlan"; graph only, like mk_graph_plan).  An
 * op publishes outputs (mk_pair_pub); an edge reads one publication of an
 * earlier op under a strategy.  The region of producer tile c along region dim
 * r is c[map[r]] / div[r] (0 where map[r] is -1); tile c publishes only where
 * c[a] == sel[a] for every axis a with sel[a] >= 0 (e.g. the last split of a
 * split-K op, which finishes the output tile).  A consumer tile c reads region
 * c[map[r]] / div[r] of the edge's publication.  Every region some consumer
 * reads becomes one event; each publishing tile adds 1; the threshold is the
 * number of publishing tiles.  Strategies (host checks only; the device sees
 * counters): MK_PAIR_WHOLE needs one region published by every tile;
 * MK_PAIR_TILE one publishing tile per region; MK_PAIR_TILE_COVER several
 * disjoint tiles covering a region; MK_PAIR_TILE_REDUCE several partials of a
 * region, the same count in every region the edge reads.  An instruction
 * waits on at most two events and signals at most two (one per publication).
 * Tasks are listed op by op in row-major grid order (last axis fastest),
 * events numbered in the order consumers first wait on them, and task t goes
 * to queue t % num_cus at slot t / num_cus.  event_first/last span each
 * event's waiting tasks (not contiguous in general).  Errors: MK_E_INVALID for
 * null/out-of-range arguments, an edge reading a later op, a strategy whose
 * check fails, a region without publishing tiles, more than two waits or
 * signals on one task (mk_last_error names the edge or task). */
enum { MK_PAIR_WHOLE = 0, MK_PAIR_TILE = 1, MK_PAIR_TILE_COVER = 2, MK_PAIR_TILE_REDUCE = 3 };
typedef struct {
  int32_t op;
  int32_t map[3], div[3], sel[3];
} mk_pair_pub;
typedef struct {
  int32_t pub, cons, strategy;
  int32_t map[3], div[3];
} mk_pair_edge;
mk_status mk_pair_plan(const mk_graph_op* ops, int32_t n_ops, const mk_pair_pub* pubs, int32_t n_pubs,
                       const mk_pair_edge* edges, int32_t n_edges, int32_t num_cus, mk_plan** out);

/* Host views of the plan's schedule metadata, valid until mk_plan_free
 * (MegaRTP article, section 4 "KernelPlan": the [num_CUs, max_len, 32] int32
 * instruction tensor, per-event thresholds).
 * queue: int32 [num_cus][max_len][32] (word layout: 0 opcode, 1 spec_id,
 *   2 operand row, 3 wait count, 4 wait event, 5 wait target per run, 6 signal
 *   count, 7 signal event, 8 signal increment, 9 task id, 10 layer, 11-13 grid
 *   coordinates, 14-23 op payload, 24/25 second wait event and target,
 *   26/27 second signal event and increment, 28/29 publication of signal 1/2
 *   (pairing plans; the device does not read them), 30-31 zero; word 3 / 6
 *   count the waits / signals (0..2); NoOp rows are all zero).
 * event_target/first/last: per event, triggers per run and the [first, last)
 *   task-id range of its successors.  task_trigger/task_wait: per task, the
 *   event it triggers / waits on, or -1; task_trigger2/task_wait2 the second
 *   ones (pairing plans), or -1.  op_table: int32 [num_ops][8] rows
 *   (opcode, spec, layer, grid x, y, z, tasks, 0).  edge_kept: per input edge, 0
 *   when dropped as residual.
 *   tile_opts: the tile options the plan was built with, defaults resolved:
 *   num_cus, gemv_rows, gateup_outs, down_rows, lm_rows, attn_splits (zeros
 *   for GLM and graph plans).  op_slots: the operand table's layout, int32
 *   [num_ops][16]: the kind (MK_SLOT_*) of the tensor each slot of an op's row
 *   points at, 0 for an unused slot (the row itself holds the addresses; one
 *   row per op, shared by all of its tile instructions: MegaRTP article,
 *   section 4, "OperandPtrTable").  pairing, attn_order: the planner choices
 *   the plan was built with, defaults resolved (pairing 0/1; attn_order 1
 *   longest first, 0 plan order; 1 and 0 for mk_pair_plan plans).
 *   At batch > 1 the matrix-core tiles read their inputs pre-split: per
 *   8-element chunk and sequence 32 bytes, the chunk's bf16 parts h = bf16(v)
 *   then bf16(v - h) (MK_SLOT_ATTN_OUT and MK_SLOT_FFN_ACT hold only this
 *   form then); the O projection and down also store the next op's normed
 *   input in this form (MK_SLOT_SPLIT_FFN: x times the FFN norm weight;
 *   MK_SLOT_SPLIT_ATTN: x times the next layer's attention norm weight, or
 *   the final norm weight for the LM head) with the sums of squares of x per
 *   chunk, fp32 [chunks][batch] (MK_SLOT_SUMSQ_*). */
enum {
  MK_SLOT_NONE = 0,
  /* weights (Llama family) */
  MK_SLOT_ATTN_NORM = 1, MK_SLOT_WQ, MK_SLOT_WK, MK_SLOT_WV, MK_SLOT_Q_NORM, MK_SLOT_K_NORM, MK_SLOT_WO,
  MK_SLOT_FFN_NORM, MK_SLOT_W_GATE, MK_SLOT_W_UP, MK_SLOT_W_DOWN, MK_SLOT_EMBED, MK_SLOT_FINAL_NORM,
  MK_SLOT_LM_HEAD,
  /* caller inputs and caches */
  MK_SLOT_TOKENS = 20, MK_SLOT_K_CACHE, MK_SLOT_V_CACHE,
  /* plan-owned data */
  MK_SLOT_ROPE = 30, MK_SLOT_QKV, MK_SLOT_ATTN_PART, MK_SLOT_ATTN_OUT, MK_SLOT_HIDDEN_ATTN, MK_SLOT_HIDDEN_FFN,
  MK_SLOT_FFN_ACT, MK_SLOT_LOGITS, MK_SLOT_LM_MAX, MK_SLOT_NEXT_TOKEN, MK_SLOT_SPLIT_ATTN, MK_SLOT_SPLIT_FFN,
  MK_SLOT_SUMSQ_ATTN, MK_SLOT_SUMSQ_FFN,
  /* the GLM pre-attention path: inputs, weights (codes, scales), caches,
     intermediates and outputs */
  MK_SLOT_G_X = 50, MK_SLOT_G_R, MK_SLOT_G_ATTN_NORM, MK_SLOT_G_W, MK_SLOT_G_W_SCALE, MK_SLOT_G_Q_A_NORM,
  MK_SLOT_G_KV_A_NORM, MK_SLOT_G_KV_CACHE, MK_SLOT_G_IDX_CACHE, MK_SLOT_G_ROWS, MK_SLOT_G_R_OUT, MK_SLOT_G_NORM,
  MK_SLOT_G_ACT, MK_SLOT_G_ACT_SCALE, MK_SLOT_G_QKVA, MK_SLOT_G_QA, MK_SLOT_G_QA_SCALE, MK_SLOT_G_Q,
  MK_SLOT_G_QIDX, MK_SLOT_G_GATE, MK_SLOT_G_GATE_PART
};
typedef struct {
  int32_t num_cus, max_len, num_tasks, num_events, num_ops, num_edges;
  const int32_t* queue;
  const uint32_t* event_target;
  const int32_t* event_first;
  const int32_t* event_last;
  const int32_t* task_trigger;
  const int32_t* task_wait;
  const int32_t* op_table;
  const uint8_t* edge_kept;
  int32_t tile_opts[6];
  const int32_t* op_slots;
  const int32_t* task_trigger2;
  const int32_t* task_wait2;
  int32_t pairing, attn_order;
} mk_plan_view;
mk_status mk_plan_export(const mk_plan* plan, mk_plan_view* out);

/* Weights: device pointers.  layer_ptrs is a HOST array of n_layers * 11 device
 * pointers in slot order (attn_norm, wq, wk, wv, q_norm, k_norm, wo, ffn_norm,
 * w_gate, w_up, w_down); q_norm/k_norm may be NULL without qk_norm.  embed and
 * final_norm are required; lm_head is ignored when tied.  All bf16. */
#define MK_LAYER_SLOTS 11
/* MK_ARCH_GLM_PREATTN: layer_ptrs holds MK_GLM_SLOTS device pointers in slot
 * order (attn_norm bf16 [hidden], w_qkva codes, s_qkva scales, w_gate, s_gate,
 * w_idxk, s_idxk, q_a_norm bf16 [q_lora], kv_a_norm bf16 [kv_lora], w_qb, s_qb,
 * w_idxq, s_idxq); embed, final_norm and lm_head are ignored. */
#define MK_GLM_SLOTS 13
typedef struct {
  const void* const* layer_ptrs;
  const void* embed;
  const void* final_norm;
  const void* lm_head;
} mk_weights;

/* Run one decode step as the persistent megakernel: ONE launch of 'num_cus'
 * workgroups on 'stream' (a hipStream_t; NULL = default stream).  Defined by:
 * CMU 15-779 lecture 7 notes, section 4.1 (the worker loop: fetch, prefetch
 * weights before waiting, wait for counters, compute, signal) and section 6
 * (the decode step's operator chain); MegaRTP article, section 4 ("Device-side
 * execution": controller / loader / consumer / storer roles, shared-memory
 * pages recycled across instructions, global event counters).
 * kv_cache: device bf16 [n_layers][2][batch][n_kv_heads][max_kv_len][head_dim];
 *   row kv_len[b] of every (layer, K|V, b, head) is written, rows < kv_len[b]
 *   are read, nothing else is touched, so repeated runs are idempotent.
 * tokens: device int32 [batch], input token ids in [0, vocab).  An id outside
 *   it fails the run: the step computes on the id clamped into range (no access
 *   leaves the embedding) and mk_plan_check returns MK_E_INVALID.
 * MK_ARCH_GLM_PREATTN: tokens is device bf16 [2][batch][hidden] (x, then r);
 *   kv_cache is device bf16, the KV cache [n_seq][max_kv_len][kv_lora +
 *   rope_dim] followed by the indexer cache [n_seq][max_kv_len][idx_head_dim]
 *   (n_seq = ceil(batch / rows_per_seq)); only row kv_len[m] of request
 *   m / rows_per_seq is written in each.
 * Results stay in the plan (see mk_plan_output).  Only enqueues work; the
 * first call uploads the plan; pointer changes rewrite the operand table.
 * A device wait that exceeds the plan's bound makes the grid exit early and is
 * reported by mk_plan_check.  The launch carries the run's epoch, so it must not
 * be captured into a graph: under stream capture mk_run returns
 * MK_E_UNSUPPORTED (capture mk_run_layerwise instead).  Errors: MK_E_INVALID,
 * MK_E_STATE (graph-only plan), MK_E_UNSUPPORTED (capture; the grid cannot be
 * co-resident on the device), MK_E_HIP. */
mk_status mk_run(mk_plan* plan, const mk_weights* weights, void* kv_cache, const void* tokens, void* stream);

/* The same step with one kernel launch per operator (stream order replaces the
 * event counters; same tiles and tile arithmetic, weights read straight from
 * memory).  The baseline the megakernel is measured against: CMU 15-779 lecture
 * 7 notes, section 2 (one kernel per operator: launch gaps, latency, tails);
 * MegaRTP article, sections 1 and 5 (fused per-op kernels on one stream; graph
 * + multistream).  It may be captured into a graph (the launch arguments
 * carry nothing that changes between runs). */
mk_status mk_run_layerwise(mk_plan* plan, const mk_weights* weights, void* kv_cache, const void* tokens,
                           void* stream);

/* Move a Llama-family plan to new sequence lengths (the next decode step)
 * without replanning (MegaRTP article, §三/§四: a plan is regenerated only when
 * tile counts or thresholds change).  Only the attention tasks' payloads (split
 * ranges and the new position) and the RoPE table depend on the lengths; the
 * queue's shape, events and targets do not, and counters stay epoch-based.  The
 * placement of the attention tasks is kept (with attn_order longest first, the
 * order chosen for the lengths the plan was built with; any placement within
 * a run of equal waits keeps every dependency).
 * kv_len: host int32 [batch], each kv_len[b] + 1 <= max_kv_len.  If the plan has
 * run, the patch is enqueued on stream (a copy from pinned host memory and a
 * small kernel that rewrites the words in the device queue) before any later
 * work on that stream; otherwise the first run uploads the patched plan.
 * mk_plan_export shows the new payloads.  Errors: MK_E_INVALID (null),
 * MK_E_STATE (graph-only plan), MK_E_UNSUPPORTED (GLM plan, a length past the
 * capacity, or an attention split that no longer fits the LDS page ring --
 * never for batched head_dim-64 plans, whose attention streams through the
 * ring: build a new plan), MK_E_HIP. */
mk_status mk_plan_set_kv_len(mk_plan* plan, const int32_t* kv_len, void* stream);

/* n_steps decode steps back to back on stream: step k runs at lengths
 * kv_len + k (kv_len: the plan's current lengths), writes its K/V rows at those
 * positions, and reads as its tokens those of step k - 1's argmax (step 0:
 * tokens, device int32 [batch]; the plan keeps its own copy).  out_tokens
 * (device int32 [n_steps][batch], or null) receives every step's next tokens.
 * layerwise != 0 runs each step as mk_run_layerwise does.  Afterwards the plan
 * is at the last step's lengths and its outputs are the last step's.  Only
 * enqueues work (the host waits at most for the upload of the call before the
 * previous one); calls on one plan must be ordered on one stream, as its runs
 * share the plan's queue and workspace.
 * Not capturable (MK_E_UNSUPPORTED under stream capture), as mk_run.
 * Defined by: CMU 15-779 lecture 7 notes, section 4.1 (the decode loop);
 * MegaRTP article, section 4 (a plan is rebuilt only when tile counts or
 * thresholds change).
 * Errors: as mk_run and mk_plan_set_kv_len; MK_E_INVALID for n_steps < 1. */
mk_status mk_run_steps(mk_plan* plan, const mk_weights* weights, void* kv_cache, const void* tokens,
                       int32_t n_steps, void* out_tokens, int32_t layerwise, void* stream);

/* Device pointer and size of a plan output (the tensors the pages' decode step
 * produces: CMU 15-779 lecture 7 notes, section 6; MegaRTP article, section 1):
 * MK_OUT_LOGITS fp32 [batch][vocab]; MK_OUT_NEXT_TOKEN int32 [batch];
 * MK_OUT_QKV fp32 [n_layers] slices of [batch][n_kv_heads][(n_q/n_kv + 2) *
 *   head_dim] (per kv head: its q heads, then k, then v, before RoPE);
 * MK_OUT_HIDDEN fp32 [n_layers][2] slices of [hidden / 8][batch][8] (residual
 *   stream after the attention block and after the FFN block of each layer;
 *   element (b, k) at ((k / 8) * batch + b) * 8 + k % 8, which at batch 1 is
 *   the plain vector); each slice of these two starts at a multiple of 256
 *   bytes (slice stride = its size rounded up to 256 bytes).
 * GLM: MK_OUT_GLM_R bf16 [M][hidden] (x + r); MK_OUT_GLM_Q bf16 [M][n_q_heads]
 *   [head_dim]; MK_OUT_GLM_QIDX bf16 [M][n_idx_heads][idx_head_dim];
 *   MK_OUT_GLM_GATE fp32 [M][n_gate]; and the intermediates MK_OUT_GLM_NORM fp32
 *   [M][hidden], MK_OUT_GLM_ACT (E4M3 codes, uint8 [M][hidden]),
 *   MK_OUT_GLM_ACT_SCALE fp32 [M][hidden/128], MK_OUT_GLM_QKVA fp32 [M][q_lora
 *   + kv_lora + rope_dim], MK_OUT_GLM_QA uint8 [M][q_lora], MK_OUT_GLM_QA_SCALE
 *   fp32 [M][q_lora/128]. */
enum { MK_OUT_LOGITS = 0, MK_OUT_NEXT_TOKEN = 1, MK_OUT_QKV = 2, MK_OUT_HIDDEN = 3 };
enum {
  MK_OUT_GLM_R = 4, MK_OUT_GLM_Q = 5, MK_OUT_GLM_QIDX = 6, MK_OUT_GLM_GATE = 7, MK_OUT_GLM_NORM = 8,
  MK_OUT_GLM_ACT = 9, MK_OUT_GLM_ACT_SCALE = 10, MK_OUT_GLM_QKVA = 11, MK_OUT_GLM_QA = 12, MK_OUT_GLM_QA_SCALE = 13
};
mk_status mk_plan_output(const mk_plan* plan, int32_t which, void** dev_ptr, size_t* bytes);
/* Enqueue a device-to-device copy of output 'which' into dst (device, at least
 * 'bytes' = the output's size) on 'stream'. */
mk_status mk_plan_copy_output(const mk_plan* plan, int32_t which, void* dst, size_t bytes, void* stream);

/* Synchronize the stream, then read back the device state of the last run
 * (MegaRTP article, section 4: every counter reaches its threshold):
 * counters_ok = 1 when every event counter equals epoch * target; err_* is the
 * watchdog record (err_kind 0 = none, 1 = event wait, 2 = page wait, 3 = ready
 * wait, 4 = drain wait, 5 = free-page wait).  Returns MK_E_TIMEOUT when the
 * record is set (the next run then clears the counters and restarts at epoch
 * 1), MK_E_INVALID when the last run's input tokens held an id outside [0,
 * vocab).  Counters are cleared the same way when they disagree with their
 * targets, and before the epoch would wrap. */
typedef struct {
  uint32_t epoch;
  int32_t counters_ok;
  int32_t bad_counters;
  int32_t err_kind, err_cu, err_slot, err_event;
  uint32_t err_value, err_target;
} mk_check;
mk_status mk_plan_check(mk_plan* plan, void* stream, mk_check* out);

/* Per-instruction timestamps of the next mk_run calls (enable=1) or none
 * (enable=0), for the active-CU fraction and bubble analysis of the MegaRTP
 * article, sections 1 and 6.  mk_plan_trace copies the last run's trace to host memory:
 * uint64 [num_cus][max_len][16] = (event satisfied, compute start, compute end,
 * signalled, first page DMA issued, last page landed in LDS, compute wave 0
 * activation ready, 0, then per compute wave 0..3 its start and its
 * pages-released time), in ticks of the device's constant clock, whose rate
 * (hipDeviceAttributeWallClockRate) is returned in ticks_per_us. */
mk_status mk_plan_set_trace(mk_plan* plan, int32_t enable);
mk_status mk_plan_trace(mk_plan* plan, void* stream, uint64_t* host_out, size_t bytes, double* ticks_per_us);

void mk_plan_free(mk_plan* plan);

/* Fill the plan's workspace (every intermediate and output) with 0xFF bytes
 * (NaN as fp32) on the stream, so that a run that read data no task of it wrote
 * shows NaN.  Errors: MK_E_STATE before the plan's first run. */
mk_status mk_plan_poison_workspace(mk_plan* plan, void* stream);

/* For tests of the watchdog: add delta to the wait threshold of the
 * instructions that wait on 'event' (re-uploaded at once if the plan has run):
 * slot 0 raises every such wait, 1 only those in an instruction's first wait,
 * 2 only those in its second wait (pairing plans).  A threshold above the
 * event's producer count makes its waiters time out: the grid drains and exits
 * normally and mk_plan_check reports MK_E_TIMEOUT.  Errors: MK_E_INVALID for an
 * event or slot out of range, MK_E_STATE for graph-only plans. */
mk_status mk_plan_debug_raise_wait(mk_plan* plan, int32_t event, int32_t delta, int32_t slot);

/* Measurement: one streaming read of 'bytes' (a multiple of 16 KiB) at src
 * (device), the ceiling a weight stream can reach on this device: 16 KiB pages
 * dealt round-robin to 'waves' waves (1..8) of each of 'workgroups' workgroups,
 * read with LDS-DMA into an LDS ring (lds_dma = 1, as the megakernel's loaders
 * do; depth 1..4 pages in flight per wave) or with 16-byte register loads
 * (lds_dma = 0; depth 1..2).  sink: device, at least workgroups * waves uint32
 * (written so the register loads are kept).  Only enqueues. */
mk_status mk_stream_probe(const void* src, size_t bytes, int32_t lds_dma, int32_t workgroups, int32_t waves,
                          int32_t depth, void* sink, void* stream);

/* mk_run for callers that cannot allocate device memory (code under graph
 * capture elsewhere in the process, tight serving loops, harnesses that forbid
 * hipMalloc): the plan's queue, counters, watchdog record, operand table, RoPE
 * table and workspace live in one static device buffer of the library (64 MiB
 * per GPU, held from first use until the process ends), and the step's outputs
 * go to the caller's buffers: logits device fp32 [batch][vocab], next_tokens
 * device int32 [batch].  It never calls hipMalloc or hipFree.  Llama-family
 * plans only; a plan whose state exceeds the buffer (see mk_noalloc_bytes) gets
 * MK_E_UNSUPPORTED.  Every call on one GPU shares that buffer and leaves its
 * contents there: the queue and RoPE table are copied in when another plan (or
 * another state of this plan) used it last, and the counters and watchdog
 * record are cleared on the stream at every call.  Calls that overlap on one
 * GPU (on different streams, or from different threads without ordering) race
 * on the buffer and give undefined results.  mk_plan_check and mk_plan_output
 * do not see these runs.  Not capturable (MK_E_UNSUPPORTED under capture). */
mk_status mk_run_noalloc(mk_plan* plan, const mk_weights* weights, void* kv_cache, const void* tokens, void* logits,
                         void* next_tokens, void* stream);
/* Bytes of the static buffer a plan needs (0 for plans mk_run_noalloc does not
 * run), and the buffer's size. */
mk_status mk_noalloc_bytes(const mk_plan* plan, size_t* need, size_t* limit);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
