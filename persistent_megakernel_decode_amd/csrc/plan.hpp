// Host-side tile planner of the persistent megakernel (no HIP dependency).
//
// Operator DAG -> tasks (tiles) -> events -> linearized task order -> static
// per-CU queues of 32-word instructions.  The rules follow the MPK internals
// notes (dpshk.com), "fine-grained pipeline" (per-dimension gcd of producer
// and consumer partitions), "handling fork producer" / "handling join
// consumer" (lcm normalization) and "building the SM-level DAG"
// (linearization: each event's successors are created contiguously), and the
// MegaRTP article (tahou.com), section 4 "KernelPlan" (round-robin placement
// into a fixed [num_CUs, max_len, 32] int32 tensor padded with NoOps).
#pragma once
#include <array>
#include <cstdint>
#include <string>
#include <vector>

namespace mk {

constexpr int kWords = 32;
constexpr int kMaxDims = 4;

// instruction words
enum : int {
  kWOpcode = 0, kWSpec = 1, kWOpRow = 2, kWWaitCnt = 3, kWWaitEv = 4, kWWaitTgt = 5,
  kWSigCnt = 6, kWSigEv = 7, kWSigInc = 8, kWTask = 9, kWLayer = 10, kWGx = 11, kWGy = 12, kWGz = 13,
  kWPay = 14, kNPay = 10,
  // second wait and second signal, and the publication of each signal
  // (pairing plans); word 31 stays free
  kWWait2Ev = 24, kWWait2Tgt = 25, kWSig2Ev = 26, kWSig2Inc = 27, kWSigPub = 28, kWSig2Pub = 29
};

// opcodes of the Llama-family decode step
enum : int { kNoop = 0, kQkv = 1, kAttn = 2, kCombine = 3, kOproj = 4, kGateUp = 5, kDown = 6, kLmHead = 7, kArgmax = 8 };
// opcodes of the GLM-style pre-attention path
enum : int { kGA0 = 9, kGQkva = 10, kGGate = 11, kGIdxk = 12, kGQaNorm = 13, kGQkvb = 14, kGIdxq = 15, kGGateRed = 16 };
constexpr int kGlmRows = 16;    // weight rows per fp8 GEMM tile
constexpr int kGateBlocks = 4;  // 128-column blocks per head-gate K-split tile (one per compute wave)

struct GraphOp {
  int opcode = 0, spec = 0, layer = 0;
  std::array<int, 3> grid{{1, 1, 1}};
  // payload words of task (x, y, z); filled by the model builder (kind-specific)
  int kind = 0;          // 0 = no payload, else opcode-specific rule
  std::array<int, 8> p{};  // parameters of the payload rule
};

struct GraphEdge {
  int prod = 0, cons = 0;
  std::array<int, 3> out_map{{-1, -1, -1}}, in_map{{-1, -1, -1}};
  bool has_extent = false;
  std::array<int, kMaxDims> extent{{1, 1, 1, 1}}, ptile{{1, 1, 1, 1}}, ctile{{1, 1, 1, 1}};
};

struct Plan {
  int num_cus = 0, max_len = 0, num_tasks = 0, num_events = 0;
  std::vector<int32_t> queue;  // [num_cus][max_len][32]
  std::vector<uint32_t> event_target;
  std::vector<int32_t> event_first, event_last;
  std::vector<int32_t> task_trigger, task_wait;    // first signal / wait per task, or -1
  std::vector<int32_t> task_trigger2, task_wait2;  // second signal / wait per task, or -1
  std::vector<std::array<int32_t, 2>> sig_pub;     // publication of each signal (pairing plans)
  std::vector<std::array<int, 4>> tasks;  // (op, x, y, z)
  std::vector<int32_t> op_table;          // [num_ops][8]
  std::vector<uint8_t> edge_kept;
};

// Returns "" on success, else an error message.  'payload' callback encodes the
// op-specific words of a task.
std::string plan_graph(const std::vector<GraphOp>& ops, const std::vector<GraphEdge>& edges, int num_cus,
                       const std::vector<int32_t>* kv_len, Plan* out);

struct ModelShape {
  int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
};
struct ModelOpts {
  int num_cus, gemv_rows, gateup_outs, down_rows, lm_rows, attn_splits;
};

// Fill 0 fields with the defaults (tiles of about 64 KiB of bf16 weights).
void resolve_opts(const ModelShape& m, const std::vector<int32_t>& kv_len, ModelOpts* o);

// Operator DAG of one Llama-family decode step, in topological order.
std::string model_graph(const ModelShape& m, int batch, const std::vector<int32_t>& kv_len, const ModelOpts& o,
                        std::vector<GraphOp>* ops, std::vector<GraphEdge>* edges);

struct GlmShape {
  int hidden, q_lora, kv_lora, rope_dim, n_heads, head_dim, n_idx_heads, idx_head_dim, n_gate;
};
// Operator DAG of the GLM-style pre-attention path for M token rows.
std::string glm_graph(const GlmShape& g, int M, std::vector<GraphOp>* ops, std::vector<GraphEdge>* edges);

// Pairing strategies (MegaRTP article, section 4, "TaskGraph").  An op
// publishes outputs; an edge reads one publication of an earlier op.  Region
// dim r of producer tile c is c[map[r]] / div[r] (0 where map[r] is -1); tile c
// publishes only if c[a] == sel[a] wherever sel[a] >= 0.  Each region some
// consumer reads is one event whose threshold is its number of publishing
// tiles.  whole: one region published by every tile; tile: one publishing tile
// per region; tile_cover: several disjoint tiles; tile_reduce: several partials,
// the same count in every region the edge reads.  At most two waits and two
// signals per instruction.  Tasks op by op in row-major grid order; events
// numbered in the order consumers first wait on them; round-robin placement.
enum : int { kPairWhole = 0, kPairTile = 1, kPairTileCover = 2, kPairTileReduce = 3 };
struct PairPub {
  int op = 0;
  std::array<int, 3> map{{-1, -1, -1}}, div{{1, 1, 1}}, sel{{-1, -1, -1}};
};
struct PairEdge {
  int pub = 0, cons = 0, strategy = kPairWhole;
  std::array<int, 3> map{{-1, -1, -1}}, div{{1, 1, 1}};
};
std::string plan_pairs(const std::vector<GraphOp>& ops, const std::vector<PairPub>& pubs,
                       const std::vector<PairEdge>& edges, int num_cus, const std::vector<int32_t>* kv_len, Plan* out);

// Publications and pairing edges of the Llama-family decode step over the ops
// model_graph lists (residual inputs kept as second waits of O and down).
void model_pairs(const std::vector<GraphOp>& ops, std::vector<PairPub>* pubs, std::vector<PairEdge>* edges);

// Longest-first placement of attention tasks within each run of consecutive
// attention tasks that wait on the same events, then re-encode the queues.
void balance_attention(const std::vector<GraphOp>& ops, const std::vector<int32_t>& kv_len, int splits, Plan* P);

inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// positions [lo, hi) of split s when pos + 1 positions are cut into S splits
inline void split_range(int pos, int S, int s, int* lo, int* hi) {
  int n = pos + 1, sz = ceil_div(n, S);
  int l = s * sz < n ? s * sz : n;
  int h = l + sz < n ? l + sz : n;
  *lo = l;
  *hi = h;
}

}  // namespace mk
