// C ABI of libmk.so (declared in include/mk.h): plan lifecycle, device
// buffers, the operand pointer table, launches, checks and traces.
//
// The operand pointer table follows the MegaRTP article, section 4
// "KernelPlan": one row of 16 u64 per operator, shared by all of its tile
// instructions, so that rebinding weights, KV cache or workspace rewrites the
// table but never the instruction queues.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_device.hpp"
#include "mk_glm.hpp"
#include "plan.hpp"

// Device memory of the allocation-free entry point (mk_run_noalloc): one
// static buffer per GPU, held from the library's load on that GPU until the
// process ends.  In host code 'scratch' names a host-side stand-in, never the
// device address: that is taken once per device with hipGetSymbolAddress
// (scratch_base) and only that address is handed to kernels and copies.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace mk {
hipError_t launch_megakernel(const mkd::KArgs& a, int num_cus, hipStream_t s);
hipError_t launch_layer(const mkd::KArgs& a, int num_cus, int first_task, int ntasks, hipStream_t s);
hipError_t megakernel_occupancy(int hd, int batch, bool glm, int* blocks_per_cu);
int ring_pages(int batch);
hipError_t launch_step_setup(int* queue, const void* patches, int n, float* rope, const float* rope_src, int nr,
                             int* tok, const int* next, int* out, int nt, hipStream_t s);
hipError_t launch_stream_probe(const void* src, long npages, int lds_dma, int workgroups, int waves, int depth,
                               unsigned* sink, hipStream_t s);
}  // namespace mk

namespace {
thread_local std::string g_err;

mk_status fail(mk_status s, const std::string& msg) {
  g_err = msg;
  return s;
}
mk_status hip_fail(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return MK_E_HIP;
}
#define HIPCHK(x, what)                          \
  do {                                           \
    hipError_t e_ = (x);                         \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)
}  // namespace

struct mk_plan {
  bool graph_only = false;
  int pairing = 0, attn_order = 0;  // planner choices of mk_plan_opts
  // identity of the plan's host state (queue words, RoPE table): uid is unique
  // per plan, version changes whenever that state is patched
  uint64_t uid = 0, version = 0;
  mk::Plan P;
  mk_model_desc desc{};
  int batch = 0;
  std::vector<int32_t> kv_len;
  mk::ModelOpts opts{};
  std::vector<mk::GraphOp> ops;
  std::vector<int> op_first, op_count;
  // layerwise baseline: an op's producers, and the stream it is launched on
  // (0: the caller's; branches of the op graph get streams of their own)
  std::vector<std::vector<int>> op_prod;
  std::vector<int> op_stream;
  int n_streams = 1;
  std::vector<hipStream_t> xs;      // [n_streams], xs[0] unused (the caller's stream)
  std::vector<hipEvent_t> op_done;  // one per op
  hipEvent_t ev_fork = nullptr;
  mkd::Consts c{};
  int num_cus = 0;
  int timeout_ms = 200;
  unsigned long long timeout_ticks = 0;  // timeout_ms in ticks of the device's constant clock
  double ticks_per_us = 100.0;           // that clock's rate (queried at upload)
  int dma_pages = 1;
  // device state
  int device = -1;
  bool uploaded = false;
  int* d_queue = nullptr;
  unsigned* d_counters = nullptr;
  unsigned* d_err = nullptr;
  uint64_t* d_optab = nullptr;
  float* d_rope = nullptr;
  char* d_ws = nullptr;
  size_t ws_bytes = 0;
  unsigned long long* d_trace = nullptr;
  bool trace_on = false;
  unsigned epoch = 0;
  unsigned run_seq = 0;  // runs of either path; a bad token id is flagged with the run's number
  bool need_reset = false;
  std::vector<uint64_t> h_optab;
  mutable std::vector<int32_t> op_slots;  // operand-table layout (MK_SLOT_* per slot), made on first export
  // new sequence lengths without replanning: the attention tasks' first words
  // in the queue, their payload patches (device and host staging) and the
  // host RoPE table
  std::vector<int> attn_words;
  int* d_patch = nullptr;
  std::vector<float> h_rope;
  // staging of a run of steps: pinned host buffer and its device copy, per step
  // the attention patches then the RoPE table; an event marks the upload.  Two
  // of them, used in turn, so that staging a call never waits for the steps the
  // previous call queued (only for the upload of the call before that)
  struct Staging {
    char* h = nullptr;
    char* d = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
  } stg[2];
  int stg_next = 0;
  int32_t* d_tok = nullptr;  // tokens of a run of steps (the previous step's next tokens)
  // workspace offsets (bytes)
  size_t off_qkv = 0, off_part = 0, off_ao = 0, off_hidden = 0, off_act = 0, off_logits = 0, off_lmmax = 0,
         off_next = 0;
  size_t sz_qkv = 0, sz_part = 0, sz_ao = 0, sz_act = 0, sz_hid = 0;
  // batch > 1: the normed GEMV inputs in pre-split form and their chunk sums of
  // squares -- QKV of layers 1..L-1 and the LM head (slices 1..L, written by
  // down), gate/up of each layer (written by O)
  size_t off_xpa = 0, off_xpf = 0, off_ssa = 0, off_ssf = 0, sz_ssc = 0;
  // GLM pre-attention path: token rows' (position, request), workspace offsets
  bool glm = false;
  int n_seq = 0;
  int* d_rows = nullptr;
  size_t off_gn = 0, off_ga8 = 0, off_gas = 0, off_gqkva = 0, off_gqa8 = 0, off_gqs = 0, off_gr = 0, off_gq = 0,
         off_gqidx = 0, off_ggate = 0, off_ggpart = 0;
};

static std::atomic<uint64_t> g_plan_uid{0};
static mk_plan* new_plan() {
  auto* p = new mk_plan();
  p->uid = ++g_plan_uid;
  return p;
}

extern "C" {

const char* mk_last_error(void) { return g_err.c_str(); }
int mk_abi_version(void) { return MK_ABI_VERSION; }

static mk_status finish_plan_common(mk_plan* p) {
  // tasks of every op must be contiguous for the layerwise launches
  const int n_ops = (int)p->ops.size();
  p->op_first.assign(n_ops, -1);
  p->op_count.assign(n_ops, 0);
  for (int t = 0; t < p->P.num_tasks; ++t) {
    int o = p->P.tasks[t][0];
    if (p->op_first[o] < 0) p->op_first[o] = t;
    if (p->op_first[o] + p->op_count[o] != t) p->op_first[o] = -2;  // not contiguous
    p->op_count[o]++;
  }
  return MK_OK;
}

// Streams of the layerwise baseline: an op continues the stream whose last op is
// one of its producers; otherwise it opens another stream (up to 3), so the
// independent branches of the op graph (the GLM path's QKV-A / gate / indexer-K
// after A0, QKV-B / indexer-Q after the q-path norm) run concurrently.  A plain
// chain (the Llama-family graph) stays on the caller's stream.
static void assign_streams(mk_plan* p, const std::vector<mk::GraphEdge>& edges, int max_streams) {
  const int n = (int)p->ops.size();
  const int kMaxStreams = std::max(1, std::min(3, max_streams));
  p->op_prod.assign(n, {});
  for (const auto& e : edges) {
    auto& v = p->op_prod[e.cons];
    if (std::find(v.begin(), v.end(), e.prod) == v.end()) v.push_back(e.prod);
  }
  p->op_stream.assign(n, 0);
  std::vector<int> tail(3, -1);
  int used = 1;
  for (int o = 0; o < n; ++o) {
    int st = -1;
    for (int q : p->op_prod[o])
      if (tail[p->op_stream[q]] == q) {
        st = p->op_stream[q];
        break;
      }
    if (st < 0) {
      if (p->op_prod[o].empty() || used == kMaxStreams) {
        // no producer (the first op), or all streams taken: the stream whose
        // last op finished earliest in program order
        st = 0;
        for (int k = 1; k < used; ++k)
          if (tail[k] < tail[st]) st = k;
        if (p->op_prod[o].empty() && tail[0] < 0) st = 0;
      } else {
        st = used++;
      }
    }
    p->op_stream[o] = st;
    tail[st] = o;
  }
  p->n_streams = used;
}

static mk_status resolve_cus(const mk_plan_opts* opts, int* num_cus, int* timeout_ms, int* dma_pages) {
  *num_cus = opts ? opts->num_cus : 0;
  if (opts && opts->timeout_ms > 0) *timeout_ms = opts->timeout_ms;
  if (opts && (opts->dma_pages < 0 || opts->dma_pages > 3))
    return fail(MK_E_INVALID, "dma_pages must be 0 (default), 1, 2 or 3");
  if (opts && opts->dma_pages > 0) *dma_pages = opts->dma_pages;
  if (opts && (opts->lw_streams < 0 || opts->lw_streams > 3)) return fail(MK_E_INVALID, "lw_streams must be 0..3");
  if (*num_cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return fail(MK_E_INVALID, "num_cus not given and no device to query");
    *num_cus = n;
  }
  return MK_OK;
}

// The GLM-style pre-attention path: fp8 weights, M <= 16 token rows.
static std::string check_cached_layout(const mk_plan* p);

static mk_status build_glm(const mk_model_desc& d, int32_t M, const int32_t* kv_len, const mk_plan_opts* opts,
                           mk_plan** out) {
  if (d.weight_dtype != MK_FP8_E4M3_B128)
    return fail(MK_E_UNSUPPORTED, "the GLM path needs E4M3 weights with 128 x 128 block scales");
  if (d.n_layers != 1) return fail(MK_E_INVALID, "the GLM path is one layer's prologue: n_layers must be 1");
  if (M < 1 || M > mkd::kMB) return fail(MK_E_UNSUPPORTED, "batch (token rows) must be 1..16");
  const int H = d.hidden, QL = d.q_lora, KL = d.kv_lora, RD = d.rope_dim, hd = d.head_dim, nh = d.n_q_heads;
  const int nope = hd - RD, Niq = d.n_idx_heads * d.idx_head_dim;
  if (d.rows_per_seq < 1 || nh < 1 || d.n_idx_heads < 1) return fail(MK_E_INVALID, "GLM sizes must be positive");
  if (H < 128 || H % 128 || QL < 128 || QL % 128) return fail(MK_E_UNSUPPORTED, "hidden and q_lora must be multiples of 128");
  if (KL < 8 || KL % 8) return fail(MK_E_UNSUPPORTED, "kv_lora must be a positive multiple of 8");
  // the row ops keep a wave's share of a row in registers (hidden: 16 blocks of
  // 128 per wave; q_lora: 8 blocks per wave over three waves; kv_lora: 2 chunks
  // of 8 per lane), and the cache rows are stored 16 bytes at a time
  if (H > mkd::kNW * 4 * mkd::kA0Groups * 128 || QL > 3 * 4 * mkd::kQaGroups * 128 || KL > 8 * 64 * mkd::kKvChunks ||
      mk::ceil_div(H / 128, mk::kGateBlocks) > mkd::kMaxGateSplits ||
      (KL + RD) % 8)
    return fail(MK_E_UNSUPPORTED, "hidden <= 8192, q_lora <= 3072, kv_lora <= 1024 and kv_lora + rope_dim a "
                                  "multiple of 8");
  if (nope < 16 || nope % 16 || RD < 16 || RD % 16 || RD > 128)
    return fail(MK_E_UNSUPPORTED, "head_dim - rope_dim and rope_dim (<= 128) must be positive multiples of 16");
  if (d.n_gate < 16 || d.n_gate % 16 || d.idx_head_dim < 16 || d.idx_head_dim % 16 || Niq % 16)
    return fail(MK_E_UNSUPPORTED, "n_gate, idx_head_dim and n_idx_heads * idx_head_dim must be multiples of 16");
  if ((QL + KL + RD) % 4) return fail(MK_E_UNSUPPORTED, "q_lora + kv_lora + rope_dim must be a multiple of 4");
  if (16L * H > (long)mk::ring_pages(2) * mkd::kPage || 16L * QL > (long)mk::ring_pages(2) * mkd::kPage)
    return fail(MK_E_UNSUPPORTED, "a 16-row fp8 tile of hidden or q_lora columns does not fit the LDS ring (128 KiB)");
  for (int h = 0; h < nh; ++h)
    if ((h * hd + nope) / 128 != (h * hd + hd - 1) / 128)
      return fail(MK_E_UNSUPPORTED, "each head's rope rows must lie in one 128-row scale block");
  if (!(d.rms_eps > 0.f) || !(d.rope_theta > 0.f)) return fail(MK_E_INVALID, "rms_eps and rope_theta must be > 0");
  const int n_seq = (M + d.rows_per_seq - 1) / d.rows_per_seq;
  std::vector<int32_t> kl(kv_len, kv_len + M);
  for (int m = 0; m < M; ++m) {
    if (kl[m] < 0 || kl[m] >= d.max_kv_len) return fail(MK_E_UNSUPPORTED, "kv_len[m] must be in [0, max_kv_len)");
    for (int j = 0; j < m; ++j)
      if (j / d.rows_per_seq == m / d.rows_per_seq && kl[j] == kl[m])
        return fail(MK_E_INVALID, "two token rows of one request write the same cache position");
  }
  auto* p = new_plan();
  p->desc = d;
  p->batch = M;
  p->kv_len = kl;
  p->glm = true;
  p->n_seq = n_seq;
  int timeout_ms = 200;
  int ncu = 0;
  mk_status st = resolve_cus(opts, &ncu, &timeout_ms, &p->dma_pages);
  if (st != MK_OK) {
    delete p;
    return st;
  }
  p->opts.num_cus = ncu;
  if (opts && (opts->pairing || opts->attn_order)) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "pairing and attn_order apply to the Llama family only");
  }
  mk::GlmShape g{H, QL, KL, RD, nh, hd, d.n_idx_heads, d.idx_head_dim, d.n_gate};
  std::vector<mk::GraphEdge> edges;
  std::string err = mk::glm_graph(g, M, &p->ops, &edges);
  if (err.empty()) err = mk::plan_graph(p->ops, edges, ncu, &p->kv_len, &p->P);
  if (!err.empty()) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "planner: " + err);
  }
  finish_plan_common(p);
  assign_streams(p, edges, opts ? opts->lw_streams : 1);
  p->num_cus = ncu;
  mkd::Consts& c = p->c;
  c.glm = 1;
  c.H = H;
  c.B = M;
  c.cap = d.max_kv_len;
  c.nq = nh;
  c.hd = 64;  // unused by the GLM kernels
  c.eps = d.rms_eps;
  c.ql = QL;
  c.kl = KL;
  c.rd = RD;
  c.nope = nope;
  c.na = QL + KL + RD;
  c.ng = d.n_gate;
  c.nik = d.idx_head_dim;
  c.niq = Niq;
  p->timeout_ms = timeout_ms;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o2 = off;
    off += (bytes + 255) / 256 * 256;
    return o2;
  };
  p->off_gn = take((size_t)M * H * 4);
  p->off_ga8 = take((size_t)M * H);
  p->off_gas = take((size_t)M * (H / 128) * 4);
  p->off_gqkva = take((size_t)M * c.na * 4);
  p->off_gqa8 = take((size_t)M * QL);
  p->off_gqs = take((size_t)M * (QL / 128) * 4);
  p->off_gr = take((size_t)M * H * 2);
  p->off_gq = take((size_t)M * nh * hd * 2);
  p->off_gqidx = take((size_t)M * Niq * 2);
  p->off_ggate = take((size_t)M * d.n_gate * 4);
  // head-gate K-split partials: [split][row tile][16 tokens][16 rows] fp32
  const int gsplits = mk::ceil_div(H / 128, mk::kGateBlocks);
  p->off_ggpart = take((size_t)gsplits * mk::ceil_div(d.n_gate, mkd::kMB) * mkd::kMB * mkd::kMB * 4);
  p->ws_bytes = off;
  const std::string lay = check_cached_layout(p);
  if (!lay.empty()) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "workspace layout: " + lay);
  }
  *out = p;
  return MK_OK;
}

// The cached-read protocol (CohT in mk_device.hpp) reads a buffer through the
// caches only when no cache line of it holds data completed under two
// different events.  The workspace layout is built that way; this checks it
// for every buffer so read, per event slice: 256-byte aligned offsets and
// sizes (the attention partials, whose blocks are not aligned, are read with
// coherent loads and are exempt).  Returns "" or what breaks the invariant.
static std::string check_cached_layout(const mk_plan* p) {
  auto al = [](size_t v) { return v % 256 == 0; };
  if (p->glm) {
    const size_t offs[] = {p->off_gn, p->off_ga8, p->off_gas, p->off_gqkva, p->off_gqa8, p->off_gqs,
                           p->off_gr, p->off_gq, p->off_gqidx, p->off_ggate, p->off_ggpart};
    for (size_t o : offs)
      if (!al(o)) return "a GLM buffer does not start on a 256-byte boundary";
    // gate partials: one 16 x 16 fp32 block (1 KiB) per (split, row tile), each its own event
    if ((size_t)mkd::kMB * mkd::kMB * 4 % 256) return "gate partial blocks are not 256-byte multiples";
    return "";
  }
  const mkd::Consts& c = p->c;
  const size_t offs[] = {p->off_qkv, p->off_ao, p->off_hidden, p->off_act, p->off_lmmax, p->off_xpa, p->off_xpf,
                         p->off_ssa, p->off_ssf, p->sz_qkv, p->sz_ao, p->sz_hid, p->sz_act, p->sz_ssc};
  for (size_t o : offs)
    if (!al(o)) return "a per-layer slice does not start on a 256-byte boundary";
  // q/k/v output: one event per kv head; its (sequence, kv head) blocks
  if (!al((size_t)c.RPG * 4)) return "a (sequence, kv head) block of the q/k/v output is not a 256-byte multiple";
  return "";
}

mk_status mk_plan_build(const mk_model_desc* desc, int32_t batch, const int32_t* kv_len, const mk_plan_opts* opts,
                        mk_plan** out) {
  g_err.clear();
  if (!desc || !kv_len || !out) return fail(MK_E_INVALID, "null argument");
  *out = nullptr;
  if (desc->abi_version != MK_ABI_VERSION || desc->struct_size != sizeof(mk_model_desc))
    return fail(MK_E_INVALID, "mk_model_desc abi_version/struct_size mismatch");
  const mk_model_desc& d = *desc;
  if (d.arch == MK_ARCH_GLM_PREATTN) return build_glm(d, batch, kv_len, opts, out);
  if (d.arch != MK_ARCH_LLAMA && d.arch != MK_ARCH_QWEN3) return fail(MK_E_UNSUPPORTED, "unknown arch");
  if (d.weight_dtype != MK_BF16) return fail(MK_E_UNSUPPORTED, "only bf16 weights are supported");
  if (d.n_layers < 1 || d.hidden < 32 || d.n_q_heads < 1 || d.n_kv_heads < 1 || d.ffn < 32 || d.vocab < 1)
    return fail(MK_E_INVALID, "model sizes must be positive");
  if (d.head_dim != 64 && d.head_dim != 128) return fail(MK_E_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d.n_q_heads % d.n_kv_heads) return fail(MK_E_UNSUPPORTED, "n_q_heads must be a multiple of n_kv_heads");
  if (d.n_q_heads / d.n_kv_heads > mkd::kNW) return fail(MK_E_UNSUPPORTED, "at most 4 query heads per kv head");
  if (d.hidden % 8 || d.ffn % 8)
    return fail(MK_E_UNSUPPORTED, "hidden and ffn must be multiples of 8");
  if (d.hidden > 8 * mkd::kNW * 64 * mkd::kMaxChunks || d.ffn > 8 * mkd::kNW * 64 * mkd::kMaxChunks ||
      d.n_q_heads * d.head_dim > 8 * mkd::kNW * 64 * mkd::kMaxChunks)
    return fail(MK_E_UNSUPPORTED, "hidden, ffn and n_q_heads*head_dim must be <= 12288");
  if ((d.arch == MK_ARCH_QWEN3) != (d.qk_norm != 0)) return fail(MK_E_INVALID, "qk_norm must match arch");
  if (!(d.rms_eps > 0.f) || !(d.rope_theta > 0.f)) return fail(MK_E_INVALID, "rms_eps and rope_theta must be > 0");
  if (batch < 1 || batch > mkd::kMB) return fail(MK_E_UNSUPPORTED, "batch must be 1..16");
  std::vector<int32_t> kl(kv_len, kv_len + batch);
  for (int b = 0; b < batch; ++b)
    if (kl[b] < 0 || kl[b] + 1 > d.max_kv_len) return fail(MK_E_UNSUPPORTED, "kv_len[b] + 1 must be <= max_kv_len");

  auto* p = new_plan();
  p->desc = d;
  p->batch = batch;
  p->kv_len = kl;
  mk::ModelOpts o{};
  int timeout_ms = 200;
  if (opts) {
    o.num_cus = opts->num_cus;
    o.gemv_rows = opts->gemv_rows;
    o.gateup_outs = opts->gateup_outs;
    o.down_rows = opts->down_rows;
    o.lm_rows = opts->lm_rows;
    o.attn_splits = opts->attn_splits;
    if (opts->timeout_ms > 0) timeout_ms = opts->timeout_ms;
    if (opts->dma_pages < 0 || opts->dma_pages > 3) {
      delete p;
      return fail(MK_E_INVALID, "dma_pages must be 0 (default), 1, 2 or 3");
    }
    if (opts->dma_pages > 0) p->dma_pages = opts->dma_pages;
    if (opts->lw_streams < 0 || opts->lw_streams > 3) {
      delete p;
      return fail(MK_E_INVALID, "lw_streams must be 0..3");
    }
    if (opts->pairing < 0 || opts->pairing > 1 || opts->attn_order < -1 || opts->attn_order > 1) {
      delete p;
      return fail(MK_E_INVALID, "pairing must be 0 or 1 and attn_order -1, 0 or 1");
    }
    p->pairing = opts->pairing;
  }
  // longest-first attention by default where sequences differ in length
  const int ao = opts ? opts->attn_order : 0;
  p->attn_order = ao == 0 ? (batch > 1 ? 1 : 0) : (ao > 0 ? 1 : 0);
  if (o.num_cus <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      delete p;
      return fail(MK_E_INVALID, "num_cus not given and no device to query");
    }
    o.num_cus = n;
  }
  mk::ModelShape ms{d.n_layers, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn, d.vocab};
  mk::resolve_opts(ms, kl, &o);
  if (o.gemv_rows > mkd::kMaxRows || 2 * o.gateup_outs > mkd::kMaxRows || o.down_rows > mkd::kMaxRows ||
      o.lm_rows > mkd::kMaxRows) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "tile rows must be <= 16");
  }
  // the GEMV tile shapes the batch-1 kernels instantiate (rows per tile by K:
  // each compute wave holds its share of a tile in registers); the batched
  // tiles read their weights from the ring, limited only by its size below
  if (batch == 1) {
    const int K_h = d.hidden, K_o = d.n_q_heads * d.head_dim, K_f = d.ffn;
    if (o.gemv_rows > mkd::gemv_max_rows(K_h) || o.gemv_rows > mkd::gemv_max_rows(K_o) ||
        2 * o.gateup_outs > mkd::gemv_max_rows(K_h) || o.down_rows > mkd::gemv_max_rows(K_f) ||
        o.lm_rows > mkd::gemv_max_rows(K_h)) {
      delete p;
      return fail(MK_E_UNSUPPORTED, "GEMV tile rows exceed the limit for K (16 rows up to K 2048, 8 up to 4096, "
                                    "4 beyond)");
    }
  }
  // every tile's weight bytes must fit the LDS page ring; the batched
  // head_dim-64 attention streams its K/V rows through the ring (any length)
  auto r1k = [](long v) { return (v + 1023) / 1024 * 1024; };
  const long ring = (long)mk::ring_pages(batch) * mkd::kPage;
  const int Smax = o.attn_splits;
  const int maxpos = *std::max_element(kl.begin(), kl.end()) + 1;
  const long attn_rows = mk::ceil_div(maxpos, Smax);
  const bool attn_streams = batch > 1 && d.head_dim == 64;
  if ((long)o.gemv_rows * d.hidden * 2 > ring || r1k((long)o.gateup_outs * d.hidden * 2) * 2 > ring ||
      (long)o.down_rows * d.ffn * 2 > ring || (long)o.gemv_rows * d.n_q_heads * d.head_dim * 2 > ring ||
      (long)o.lm_rows * d.hidden * 2 > ring || (!attn_streams && r1k(attn_rows * d.head_dim * 2) * 2 > ring)) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "a tile does not fit the LDS page ring (144 KiB, 128 KiB for batch > 1); use smaller tiles");
  }
  if (o.attn_splits > 64) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "at most 64 attention splits");
  }
  p->opts = o;
  std::vector<mk::GraphEdge> edges;
  std::string err = mk::model_graph(ms, batch, kl, o, &p->ops, &edges);
  if (err.empty() && p->pairing) {
    std::vector<mk::PairPub> pubs;
    std::vector<mk::PairEdge> pedges;
    mk::model_pairs(p->ops, &pubs, &pedges);
    err = mk::plan_pairs(p->ops, pubs, pedges, o.num_cus, &p->kv_len, &p->P);
  } else if (err.empty()) {
    err = mk::plan_graph(p->ops, edges, o.num_cus, &p->kv_len, &p->P);
  }
  if (err.empty() && p->attn_order) mk::balance_attention(p->ops, p->kv_len, o.attn_splits, &p->P);
  if (!err.empty()) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "planner: " + err);
  }
  finish_plan_common(p);
  assign_streams(p, edges, opts ? opts->lw_streams : 1);
  for (size_t t = 0; t * 32 < p->P.queue.size(); ++t)
    if (p->P.queue[t * 32 + mkd::WOpcode] == mkd::OpAttn) p->attn_words.push_back((int)(t * 32));
  for (size_t k = 0; k < p->ops.size(); ++k)
    if (p->op_first[k] < 0) {
      delete p;
      return fail(MK_E_UNSUPPORTED, "planner: an operator's tasks are not contiguous");
    }
  p->num_cus = o.num_cus;
  const int hpg = d.n_q_heads / d.n_kv_heads;
  mkd::Consts& c = p->c;
  c.H = d.hidden;
  c.nq = d.n_q_heads;
  c.nkv = d.n_kv_heads;
  c.hd = d.head_dim;
  c.F = d.ffn;
  c.V = d.vocab;
  c.L = d.n_layers;
  c.B = batch;
  c.cap = d.max_kv_len;
  c.hpg = hpg;
  c.RPG = (hpg + 2) * d.head_dim;
  c.S = o.attn_splits;
  c.T_v = mk::ceil_div(d.vocab, o.lm_rows);
  c.qk_norm = d.qk_norm;
  c.eps = d.rms_eps;
  c.inv_sqrt_hd = (float)(1.0 / std::sqrt((double)d.head_dim));
  // rows per stored sum of squares: the largest of 8, 4, 2, 1 that divides the
  // producing tiles' rows (down for the QKV / LM-head input, O for gate/up's)
  auto sum_rows = [](int rows) { return rows % 8 == 0 ? 8 : rows % 4 == 0 ? 4 : rows % 2 == 0 ? 2 : 1; };
  c.ssg_a = sum_rows(o.down_rows);
  c.ssg_f = sum_rows(o.gemv_rows);
  p->timeout_ms = timeout_ms;
  // workspace layout (fp32 everywhere)
  const size_t B = batch, L = d.n_layers;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o2 = off;
    off += (bytes + 255) / 256 * 256;
    return o2;
  };
  // per-layer slices start on 256-byte boundaries: no cache line holds data
  // of two layers (written under different events)
  auto r256 = [](size_t v) { return (v + 255) / 256 * 256; };
  p->sz_qkv = r256(B * c.nkv * c.RPG * 4);
  p->sz_part = r256(B * c.nkv * c.S * hpg * (c.hd + 2) * 4);
  p->sz_ao = r256(B * c.nq * c.hd * 4);
  p->sz_act = r256(B * c.F * 4);
  p->sz_hid = r256(B * c.H * 4);
  p->off_qkv = take(p->sz_qkv * L);
  p->off_part = take(p->sz_part * L);
  p->off_ao = take(p->sz_ao * L);
  p->off_hidden = take(p->sz_hid * 2 * L);
  p->off_act = take(p->sz_act * L);
  if (B > 1) {
    p->sz_ssc = r256((size_t)c.H * B * 4);  // up to one sum per row (rows per sum: ssg_a, ssg_f)
    p->off_xpa = take(p->sz_hid * (L + 1));
    p->off_xpf = take(p->sz_hid * L);
    p->off_ssa = take(p->sz_ssc * (L + 1));
    p->off_ssf = take(p->sz_ssc * L);
  }
  p->off_lmmax = take(B * c.T_v * 8);
  // the step's outputs last: the allocation-free entry point keeps everything
  // before them in its static buffer and writes the outputs to the caller's
  p->off_logits = take(B * c.V * 4);
  p->off_next = take(B * 4);
  p->ws_bytes = off;
  const std::string lay = check_cached_layout(p);
  if (!lay.empty()) {
    delete p;
    return fail(MK_E_UNSUPPORTED, "workspace layout: " + lay);
  }
  *out = p;
  return MK_OK;
}

mk_status mk_graph_plan(const mk_graph_op* ops, int32_t n_ops, const mk_graph_edge* edges, int32_t n_edges,
                        int32_t num_cus, mk_plan** out) {
  g_err.clear();
  if (!out || (n_ops > 0 && !ops) || (n_edges > 0 && !edges) || n_ops < 0 || n_edges < 0)
    return fail(MK_E_INVALID, "null argument");
  *out = nullptr;
  auto* p = new_plan();
  p->graph_only = true;
  std::vector<mk::GraphEdge> ge;
  for (int i = 0; i < n_ops; ++i) {
    mk::GraphOp op;
    op.opcode = ops[i].opcode;
    op.spec = ops[i].spec;
    op.layer = ops[i].layer;
    op.grid = {{ops[i].grid[0], ops[i].grid[1], ops[i].grid[2]}};
    p->ops.push_back(op);
  }
  for (int i = 0; i < n_edges; ++i) {
    mk::GraphEdge e;
    e.prod = edges[i].prod;
    e.cons = edges[i].cons;
    for (int a = 0; a < 3; ++a) {
      e.out_map[a] = edges[i].out_map[a];
      e.in_map[a] = edges[i].in_map[a];
    }
    e.has_extent = edges[i].has_extent != 0;
    for (int k = 0; k < 4; ++k) {
      e.extent[k] = edges[i].extent[k];
      e.ptile[k] = edges[i].ptile[k];
      e.ctile[k] = edges[i].ctile[k];
    }
    ge.push_back(e);
  }
  std::string err = mk::plan_graph(p->ops, ge, num_cus, nullptr, &p->P);
  if (!err.empty()) {
    delete p;
    return fail(MK_E_INVALID, "planner: " + err);
  }
  finish_plan_common(p);
  p->num_cus = num_cus;
  *out = p;
  return MK_OK;
}

mk_status mk_pair_plan(const mk_graph_op* ops, int32_t n_ops, const mk_pair_pub* pubs, int32_t n_pubs,
                       const mk_pair_edge* edges, int32_t n_edges, int32_t num_cus, mk_plan** out) {
  g_err.clear();
  if (!out || (n_ops > 0 && !ops) || (n_pubs > 0 && !pubs) || (n_edges > 0 && !edges) || n_ops < 0 || n_pubs < 0 ||
      n_edges < 0)
    return fail(MK_E_INVALID, "null argument");
  *out = nullptr;
  auto* p = new_plan();
  p->graph_only = true;
  p->pairing = 1;
  for (int i = 0; i < n_ops; ++i) {
    mk::GraphOp op;
    op.opcode = ops[i].opcode;
    op.spec = ops[i].spec;
    op.layer = ops[i].layer;
    op.grid = {{ops[i].grid[0], ops[i].grid[1], ops[i].grid[2]}};
    p->ops.push_back(op);
  }
  std::vector<mk::PairPub> pp(n_pubs);
  for (int i = 0; i < n_pubs; ++i) {
    pp[i].op = pubs[i].op;
    for (int r = 0; r < 3; ++r) {
      pp[i].map[r] = pubs[i].map[r];
      pp[i].div[r] = pubs[i].div[r];
      pp[i].sel[r] = pubs[i].sel[r];
    }
  }
  std::vector<mk::PairEdge> pe(n_edges);
  for (int i = 0; i < n_edges; ++i) {
    pe[i].pub = edges[i].pub;
    pe[i].cons = edges[i].cons;
    pe[i].strategy = edges[i].strategy;
    for (int r = 0; r < 3; ++r) {
      pe[i].map[r] = edges[i].map[r];
      pe[i].div[r] = edges[i].div[r];
    }
  }
  std::string err = mk::plan_pairs(p->ops, pp, pe, num_cus, nullptr, &p->P);
  if (!err.empty()) {
    delete p;
    return fail(MK_E_INVALID, "planner: " + err);
  }
  finish_plan_common(p);
  p->num_cus = num_cus;
  *out = p;
  return MK_OK;
}

// kCtrSub sub-counter lines per event
static size_t counter_bytes(const mk_plan* p) {
  return (size_t)mkd::kCtrSub * std::max(1, p->P.num_events) * mkd::kCtrStride * 4;
}

// RoPE table (cos, sin) at each sequence's (GLM: token row's) new position,
// computed in fp64; rotate-half over the rope width
static void rope_table(mk_plan* p) {
  const int rope_w = p->glm ? p->c.rd : p->c.hd;
  p->h_rope.assign((size_t)p->batch * rope_w, 0.f);
  const int half = rope_w / 2;
  for (int b = 0; b < p->batch; ++b)
    for (int i = 0; i < half; ++i) {
      double ang = (double)p->kv_len[b] * std::pow((double)p->desc.rope_theta, -2.0 * i / rope_w);
      p->h_rope[(size_t)b * rope_w + 2 * i] = (float)std::cos(ang);
      p->h_rope[(size_t)b * rope_w + 2 * i + 1] = (float)std::sin(ang);
    }
}

static mk_status ensure_device(mk_plan* p) {
  if (p->uploaded) {
    int dev = -1;
    HIPCHK(hipGetDevice(&dev), "hipGetDevice");
    if (dev != p->device) return fail(MK_E_STATE, "plan was uploaded to another device");
    return MK_OK;
  }
  HIPCHK(hipGetDevice(&p->device), "hipGetDevice");
  // the device's constant-rate clock (s_memrealtime), in kHz: trace ticks and
  // the watchdog bound are counted in it
  int clk_khz = 0;
  HIPCHK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, p->device), "hipDeviceGetAttribute clock");
  if (clk_khz <= 0) return fail(MK_E_HIP, "the device reports no constant clock rate");
  p->ticks_per_us = clk_khz / 1000.0;
  p->timeout_ticks = (unsigned long long)p->timeout_ms * (unsigned long long)clk_khz;
  int ncu = 0;
  HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, p->device), "hipDeviceGetAttribute");
  int occ = 0;
  HIPCHK(mk::megakernel_occupancy(p->c.hd, p->batch, p->c.glm != 0, &occ), "occupancy");
  if (p->num_cus > ncu || occ < 1)
    return fail(MK_E_UNSUPPORTED, "the persistent grid (" + std::to_string(p->num_cus) + " workgroups) cannot be co-resident on " +
                                      std::to_string(ncu) + " CUs");
  const size_t qbytes = p->P.queue.size() * 4, ebytes = counter_bytes(p);
  HIPCHK(hipMalloc(&p->d_queue, qbytes), "hipMalloc queue");
  HIPCHK(hipMalloc(&p->d_counters, ebytes), "hipMalloc counters");
  HIPCHK(hipMalloc(&p->d_err, 64), "hipMalloc err");
  HIPCHK(hipMalloc(&p->d_optab, p->ops.size() * 16 * 8), "hipMalloc optab");
  const int rope_w = p->glm ? p->c.rd : p->c.hd;  // (cos, sin) pairs per row
  HIPCHK(hipMalloc(&p->d_rope, (size_t)p->batch * rope_w * 4), "hipMalloc rope");
  HIPCHK(hipMalloc(&p->d_ws, p->ws_bytes), "hipMalloc workspace");
  HIPCHK(hipMemcpy(p->d_queue, p->P.queue.data(), qbytes, hipMemcpyHostToDevice), "upload queue");
  HIPCHK(hipMemset(p->d_counters, 0, ebytes), "zero counters");
  HIPCHK(hipMemset(p->d_err, 0, 64), "zero err");
  HIPCHK(hipMemset(p->d_ws, 0xFF, p->ws_bytes), "poison workspace");  // NaN until written
  rope_table(p);
  HIPCHK(hipMemcpy(p->d_rope, p->h_rope.data(), p->h_rope.size() * 4, hipMemcpyHostToDevice), "upload rope");
  if (!p->glm) {
    HIPCHK(hipMalloc(&p->d_patch, std::max<size_t>(1, p->attn_words.size()) * 16), "hipMalloc patches");
  }
  if (p->glm) {
    // token rows: cache position, then request
    std::vector<int32_t> rows(2 * (size_t)p->batch);
    for (int m = 0; m < p->batch; ++m) {
      rows[m] = p->kv_len[m];
      rows[p->batch + m] = m / p->desc.rows_per_seq;
    }
    HIPCHK(hipMalloc(&p->d_rows, rows.size() * 4), "hipMalloc rows");
    HIPCHK(hipMemcpy(p->d_rows, rows.data(), rows.size() * 4, hipMemcpyHostToDevice), "upload rows");
  }
  p->uploaded = true;
  p->epoch = 0;
  return MK_OK;
}

// Where a run's plan-owned device data lives: the plan's own buffers (mk_run,
// mk_run_layerwise) or the library's static buffer (mk_run_noalloc).  cache is
// the host copy of what the device operand table holds.
struct Bind {
  char* ws;
  float* rope;
  float* logits;
  int* next;
  uint64_t* optab;
  std::vector<uint64_t>* cache;
};
static Bind own_bind(mk_plan* p) {
  return Bind{p->d_ws, p->d_rope, (float*)(p->d_ws + p->off_logits), (int*)(p->d_ws + p->off_next), p->d_optab,
              &p->h_optab};
}

static mk_status upload_optab(const Bind& b, const std::vector<uint64_t>& t, hipStream_t s) {
  if (t != *b.cache) {
    *b.cache = t;
    HIPCHK(hipMemcpyAsync(b.optab, b.cache->data(), t.size() * 8, hipMemcpyHostToDevice, s), "upload operand table");
    HIPCHK(hipStreamSynchronize(s), "operand table sync");
  }
  return MK_OK;
}

// Everything an operand row can point at.  Fields may be null when only the
// table's layout (the slot kinds) is wanted.
struct Src {
  const void* const* layer_ptrs = nullptr;
  const void* embed = nullptr;
  const void* final_norm = nullptr;
  const void* lm_head = nullptr;
  const void* kv = nullptr;
  const void* tokens = nullptr;
  Bind b{};
};

// The operand table: one row of 16 slots per op (MegaRTP article, section 4,
// "OperandPtrTable"); vals gets the addresses, kinds the MK_SLOT_* of each
// slot (0 where unused).
static void fill_rows(const mk_plan* p, const Src& src, uint64_t* vals, int32_t* kinds) {
  const mk_model_desc& d = p->desc;
  auto u = [](const void* q) { return (uint64_t)(uintptr_t)q; };
  auto ws = [&](size_t off) { return src.b.ws ? (uint64_t)(uintptr_t)(src.b.ws + off) : (uint64_t)0; };
  auto put = [&](size_t o, int slot, uint64_t v, int kind) {
    vals[o * 16 + slot] = v;
    kinds[o * 16 + slot] = kind;
  };
  std::fill(vals, vals + p->ops.size() * 16, (uint64_t)0);
  std::fill(kinds, kinds + p->ops.size() * 16, 0);
  if (p->glm) {
    const void* const* W = src.layer_ptrs;
    auto w = [&](int k) { return W ? u(W[k]) : (uint64_t)0; };
    const size_t M = p->batch, H = d.hidden;
    const uint64_t x = u(src.tokens), r = src.tokens ? u((const char*)src.tokens + M * H * 2) : 0;
    const uint64_t kvc = u(src.kv);
    const uint64_t idc =
        src.kv ? u((const char*)src.kv + (size_t)p->n_seq * d.max_kv_len * (d.kv_lora + d.rope_dim) * 2) : 0;
    for (size_t o = 0; o < p->ops.size(); ++o) {
      switch (p->ops[o].opcode) {
        case mk::kGA0:
          put(o, mkd::GaX, x, MK_SLOT_G_X);
          put(o, mkd::GaR, r, MK_SLOT_G_R);
          put(o, mkd::GaNorm, w(0), MK_SLOT_G_ATTN_NORM);
          put(o, mkd::GaROut, ws(p->off_gr), MK_SLOT_G_R_OUT);
          put(o, mkd::GaN, ws(p->off_gn), MK_SLOT_G_NORM);
          put(o, mkd::GaA8, ws(p->off_ga8), MK_SLOT_G_ACT);
          put(o, mkd::GaAS, ws(p->off_gas), MK_SLOT_G_ACT_SCALE);
          break;
        case mk::kGQkva:
          put(o, mkd::GmW, w(1), MK_SLOT_G_W);
          put(o, mkd::GmS, w(2), MK_SLOT_G_W_SCALE);
          put(o, mkd::GmA8, ws(p->off_ga8), MK_SLOT_G_ACT);
          put(o, mkd::GmAS, ws(p->off_gas), MK_SLOT_G_ACT_SCALE);
          put(o, mkd::GmOut, ws(p->off_gqkva), MK_SLOT_G_QKVA);
          break;
        case mk::kGGate:
          put(o, mkd::GmW, w(3), MK_SLOT_G_W);
          put(o, mkd::GmS, w(4), MK_SLOT_G_W_SCALE);
          put(o, mkd::GmAF, ws(p->off_gn), MK_SLOT_G_NORM);
          put(o, mkd::GmOut, ws(p->off_ggpart), MK_SLOT_G_GATE_PART);
          break;
        case mk::kGGateRed:
          put(o, mkd::GrPart, ws(p->off_ggpart), MK_SLOT_G_GATE_PART);
          put(o, mkd::GrOut, ws(p->off_ggate), MK_SLOT_G_GATE);
          break;
        case mk::kGIdxk:
          put(o, mkd::GmW, w(5), MK_SLOT_G_W);
          put(o, mkd::GmS, w(6), MK_SLOT_G_W_SCALE);
          put(o, mkd::GmA8, ws(p->off_ga8), MK_SLOT_G_ACT);
          put(o, mkd::GmAS, ws(p->off_gas), MK_SLOT_G_ACT_SCALE);
          put(o, mkd::GmOut, idc, MK_SLOT_G_IDX_CACHE);
          put(o, mkd::GmRows, u(p->d_rows), MK_SLOT_G_ROWS);
          break;
        case mk::kGQaNorm:
          put(o, mkd::QnIn, ws(p->off_gqkva), MK_SLOT_G_QKVA);
          put(o, mkd::QnNorm, w(7), MK_SLOT_G_Q_A_NORM);
          put(o, mkd::QnKvNorm, w(8), MK_SLOT_G_KV_A_NORM);
          put(o, mkd::QnA8, ws(p->off_gqa8), MK_SLOT_G_QA);
          put(o, mkd::QnAS, ws(p->off_gqs), MK_SLOT_G_QA_SCALE);
          put(o, mkd::QnKv, kvc, MK_SLOT_G_KV_CACHE);
          put(o, mkd::QnRope, u(src.b.rope), MK_SLOT_ROPE);
          put(o, mkd::QnRows, u(p->d_rows), MK_SLOT_G_ROWS);
          break;
        case mk::kGQkvb:
          put(o, mkd::GmW, w(9), MK_SLOT_G_W);
          put(o, mkd::GmS, w(10), MK_SLOT_G_W_SCALE);
          put(o, mkd::GmA8, ws(p->off_gqa8), MK_SLOT_G_QA);
          put(o, mkd::GmAS, ws(p->off_gqs), MK_SLOT_G_QA_SCALE);
          put(o, mkd::GmOut, ws(p->off_gq), MK_SLOT_G_Q);
          put(o, mkd::GmRope, u(src.b.rope), MK_SLOT_ROPE);
          break;
        case mk::kGIdxq:
          put(o, mkd::GmW, w(11), MK_SLOT_G_W);
          put(o, mkd::GmS, w(12), MK_SLOT_G_W_SCALE);
          put(o, mkd::GmA8, ws(p->off_gqa8), MK_SLOT_G_QA);
          put(o, mkd::GmAS, ws(p->off_gqs), MK_SLOT_G_QA_SCALE);
          put(o, mkd::GmOut, ws(p->off_gqidx), MK_SLOT_G_QIDX);
          break;
        default:
          break;
      }
    }
    return;
  }
  const int L = d.n_layers;
  const size_t B = p->batch;
  const size_t hid = p->sz_hid;
  auto xa = [&](int l) { return ws(p->off_hidden + (size_t)(2 * l) * hid); };
  auto xb = [&](int l) { return ws(p->off_hidden + (size_t)(2 * l + 1) * hid); };
  const bool split = B > 1;  // pre-split GEMV inputs (batched tiles)
  auto xpa = [&](int l) { return ws(p->off_xpa + (size_t)l * hid); };
  auto xpf = [&](int l) { return ws(p->off_xpf + (size_t)l * hid); };
  auto ssa = [&](int l) { return ws(p->off_ssa + (size_t)l * p->sz_ssc); };
  auto ssf = [&](int l) { return ws(p->off_ssf + (size_t)l * p->sz_ssc); };
  auto attn_norm = [&](int l) {  // layer l's attention RMSNorm weight; the final norm past the last layer
    if (l >= L) return u(src.final_norm);
    return src.layer_ptrs ? u(src.layer_ptrs[(size_t)l * MK_LAYER_SLOTS + 0]) : (uint64_t)0;
  };
  const size_t kvlayer = (size_t)2 * B * d.n_kv_heads * d.max_kv_len * d.head_dim * 2;
  auto kvp = [&](int l, int half) {
    return src.kv ? u((const char*)src.kv + l * kvlayer + half * (kvlayer / 2)) : (uint64_t)0;
  };
  for (size_t o = 0; o < p->ops.size(); ++o) {
    const auto& op = p->ops[o];
    const int l = op.layer;
    auto w = [&](int k) {
      return (src.layer_ptrs && l < L) ? u(src.layer_ptrs[(size_t)l * MK_LAYER_SLOTS + k]) : (uint64_t)0;
    };
    switch (op.opcode) {
      case mk::kQkv:
        put(o, mkd::QkvWq, w(1), MK_SLOT_WQ);
        put(o, mkd::QkvWk, w(2), MK_SLOT_WK);
        put(o, mkd::QkvWv, w(3), MK_SLOT_WV);
        put(o, mkd::QkvNorm, w(0), MK_SLOT_ATTN_NORM);
        if (l) put(o, mkd::QkvX, xb(l - 1), MK_SLOT_HIDDEN_FFN);  // layer 0 reads the embedding row
        put(o, mkd::QkvEmbed, u(src.embed), MK_SLOT_EMBED);
        put(o, mkd::QkvTokens, u(src.tokens), MK_SLOT_TOKENS);
        put(o, mkd::QkvOut, ws(p->off_qkv + l * p->sz_qkv), MK_SLOT_QKV);
        if (split && l) {
          put(o, mkd::QkvPrep, xpa(l), MK_SLOT_SPLIT_ATTN);
          put(o, mkd::QkvSs, ssa(l), MK_SLOT_SUMSQ_ATTN);
        }
        break;
      case mk::kAttn:
        put(o, mkd::AttnQkv, ws(p->off_qkv + l * p->sz_qkv), MK_SLOT_QKV);
        put(o, mkd::AttnK, kvp(l, 0), MK_SLOT_K_CACHE);
        put(o, mkd::AttnV, kvp(l, 1), MK_SLOT_V_CACHE);
        put(o, mkd::AttnRope, u(src.b.rope), MK_SLOT_ROPE);
        put(o, mkd::AttnOut, ws(p->off_part + l * p->sz_part), MK_SLOT_ATTN_PART);
        if (d.qk_norm) {
          put(o, mkd::AttnQn, w(4), MK_SLOT_Q_NORM);
          put(o, mkd::AttnKn, w(5), MK_SLOT_K_NORM);
        }
        break;
      case mk::kCombine:
        put(o, mkd::CombPart, ws(p->off_part + l * p->sz_part), MK_SLOT_ATTN_PART);
        put(o, mkd::CombOut, ws(p->off_ao + l * p->sz_ao), MK_SLOT_ATTN_OUT);
        break;
      case mk::kOproj:
        put(o, mkd::OWo, w(6), MK_SLOT_WO);
        put(o, mkd::OIn, ws(p->off_ao + l * p->sz_ao), MK_SLOT_ATTN_OUT);
        if (l) put(o, mkd::OX, xb(l - 1), MK_SLOT_HIDDEN_FFN);  // layer 0: the embedding row is the residual
        put(o, mkd::OEmbed, u(src.embed), MK_SLOT_EMBED);
        put(o, mkd::OTokens, u(src.tokens), MK_SLOT_TOKENS);
        put(o, mkd::OOut, xa(l), MK_SLOT_HIDDEN_ATTN);
        if (split) {
          put(o, mkd::OPrepW, w(7), MK_SLOT_FFN_NORM);
          put(o, mkd::OPrep, xpf(l), MK_SLOT_SPLIT_FFN);
          put(o, mkd::OSs, ssf(l), MK_SLOT_SUMSQ_FFN);
        }
        break;
      case mk::kGateUp:
        put(o, mkd::GuWg, w(8), MK_SLOT_W_GATE);
        put(o, mkd::GuWu, w(9), MK_SLOT_W_UP);
        put(o, mkd::GuNorm, w(7), MK_SLOT_FFN_NORM);
        put(o, mkd::GuIn, xa(l), MK_SLOT_HIDDEN_ATTN);
        put(o, mkd::GuOut, ws(p->off_act + l * p->sz_act), MK_SLOT_FFN_ACT);
        if (split) {
          put(o, mkd::GuPrep, xpf(l), MK_SLOT_SPLIT_FFN);
          put(o, mkd::GuSs, ssf(l), MK_SLOT_SUMSQ_FFN);
        }
        break;
      case mk::kDown:
        put(o, mkd::DnW, w(10), MK_SLOT_W_DOWN);
        put(o, mkd::DnIn, ws(p->off_act + l * p->sz_act), MK_SLOT_FFN_ACT);
        put(o, mkd::DnRes, xa(l), MK_SLOT_HIDDEN_ATTN);
        put(o, mkd::DnOut, xb(l), MK_SLOT_HIDDEN_FFN);
        if (split) {
          put(o, mkd::DnPrepW, attn_norm(l + 1), l + 1 < L ? MK_SLOT_ATTN_NORM : MK_SLOT_FINAL_NORM);
          put(o, mkd::DnPrep, xpa(l + 1), MK_SLOT_SPLIT_ATTN);
          put(o, mkd::DnSs, ssa(l + 1), MK_SLOT_SUMSQ_ATTN);
        }
        break;
      case mk::kLmHead:
        if (d.tied_lm_head)
          put(o, mkd::LmW, u(src.embed), MK_SLOT_EMBED);
        else
          put(o, mkd::LmW, u(src.lm_head), MK_SLOT_LM_HEAD);
        put(o, mkd::LmNorm, u(src.final_norm), MK_SLOT_FINAL_NORM);
        put(o, mkd::LmIn, xb(L - 1), MK_SLOT_HIDDEN_FFN);
        put(o, mkd::LmLogits, u(src.b.logits), MK_SLOT_LOGITS);
        put(o, mkd::LmMax, ws(p->off_lmmax), MK_SLOT_LM_MAX);
        if (split) {
          put(o, mkd::LmPrep, xpa(L), MK_SLOT_SPLIT_ATTN);
          put(o, mkd::LmSs, ssa(L), MK_SLOT_SUMSQ_ATTN);
        }
        break;
      case mk::kArgmax:
        put(o, mkd::AmMax, ws(p->off_lmmax), MK_SLOT_LM_MAX);
        put(o, mkd::AmOut, u(src.b.next), MK_SLOT_NEXT_TOKEN);
        break;
      default:
        break;
    }
  }
}

static mk_status bind_operands(mk_plan* p, const mk_weights* w, void* kv, const void* tokens, hipStream_t s,
                               const Bind& b) {
  const mk_model_desc& d = p->desc;
  Src src;
  src.b = b;
  src.kv = kv;
  src.tokens = tokens;
  if (p->glm) {
    if (!w || !w->layer_ptrs || !kv || !tokens) return fail(MK_E_INVALID, "null weight, cache or input pointer");
    for (int k = 0; k < MK_GLM_SLOTS; ++k)
      if (!w->layer_ptrs[k]) return fail(MK_E_INVALID, "null GLM weight pointer");
    src.layer_ptrs = w->layer_ptrs;
  } else {
    if (!w || !w->layer_ptrs || !w->embed || !w->final_norm || !kv || !tokens)
      return fail(MK_E_INVALID, "null weight, KV-cache or token pointer");
    if (!d.tied_lm_head && !w->lm_head) return fail(MK_E_INVALID, "lm_head is required when not tied");
    for (int l = 0; l < d.n_layers; ++l)
      for (int sidx = 0; sidx < MK_LAYER_SLOTS; ++sidx) {
        bool need = !(sidx == 4 || sidx == 5) || d.qk_norm;
        if (need && !w->layer_ptrs[l * MK_LAYER_SLOTS + sidx]) return fail(MK_E_INVALID, "null layer weight pointer");
      }
    src.layer_ptrs = w->layer_ptrs;
    src.embed = w->embed;
    src.final_norm = w->final_norm;
    src.lm_head = w->lm_head;
  }
  std::vector<uint64_t> t(p->ops.size() * 16, 0);
  std::vector<int32_t> kinds(p->ops.size() * 16, 0);
  fill_rows(p, src, t.data(), kinds.data());
  return upload_optab(b, t, s);
}

mk_status mk_plan_export(const mk_plan* p, mk_plan_view* v) {
  g_err.clear();
  if (!p || !v) return fail(MK_E_INVALID, "null argument");
  v->num_cus = p->P.num_cus;
  v->max_len = p->P.max_len;
  v->num_tasks = p->P.num_tasks;
  v->num_events = p->P.num_events;
  v->num_ops = (int32_t)p->ops.size();
  v->num_edges = (int32_t)p->P.edge_kept.size();
  v->queue = p->P.queue.data();
  v->event_target = p->P.event_target.data();
  v->event_first = p->P.event_first.data();
  v->event_last = p->P.event_last.data();
  v->task_trigger = p->P.task_trigger.data();
  v->task_wait = p->P.task_wait.data();
  v->op_table = p->P.op_table.data();
  v->edge_kept = p->P.edge_kept.data();
  std::fill(v->tile_opts, v->tile_opts + 6, 0);
  if (!p->graph_only && !p->glm) {
    const mk::ModelOpts& o = p->opts;
    const int32_t t[6] = {o.num_cus, o.gemv_rows, o.gateup_outs, o.down_rows, o.lm_rows, o.attn_splits};
    std::copy(t, t + 6, v->tile_opts);
  }
  if (p->op_slots.size() != p->ops.size() * 16) {
    std::vector<uint64_t> vals(p->ops.size() * 16);
    p->op_slots.assign(p->ops.size() * 16, 0);
    if (!p->graph_only) fill_rows(p, Src{}, vals.data(), p->op_slots.data());
  }
  v->op_slots = p->op_slots.data();
  v->task_trigger2 = p->P.task_trigger2.data();
  v->task_wait2 = p->P.task_wait2.data();
  v->pairing = p->pairing;
  v->attn_order = p->attn_order;
  return MK_OK;
}

static mk_status launch_step(mk_plan* p, hipStream_t s);
static mk_status launch_layerwise(mk_plan* p, hipStream_t s);

static mkd::KArgs kargs(const mk_plan* p, const int* queue, const uint64_t* optab, unsigned* counters, unsigned* err) {
  mkd::KArgs a{};
  a.queue = queue;
  a.optab = optab;
  a.counters = counters;
  a.num_events = std::max(1, p->P.num_events);
  a.err = err;
  a.trace = p->trace_on ? p->d_trace : nullptr;
  a.max_len = p->P.max_len;
  a.dma_pages = p->dma_pages;
  a.epoch = p->epoch;
  a.run_id = p->run_seq;
  a.timeout_ticks = p->timeout_ticks;
  a.c = p->c;
  return a;
}
static mkd::KArgs kargs(const mk_plan* p) { return kargs(p, p->d_queue, p->d_optab, p->d_counters, p->d_err); }

// The megakernel's launch arguments carry the run's epoch (its event waits
// compare counters with epoch * target), so a captured launch would replay a
// stale epoch: the persistent path refuses stream capture.
static mk_status refuse_capture(hipStream_t s, const char* what) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  HIPCHK(hipStreamIsCapturing(s, &cs), "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone)
    return fail(MK_E_UNSUPPORTED, std::string(what) + " cannot be captured into a graph (each run's epoch is a launch "
                                                      "argument); capture mk_run_layerwise instead");
  return MK_OK;
}

mk_status mk_run(mk_plan* p, const mk_weights* w, void* kv_cache, const void* tokens, void* stream) {
  g_err.clear();
  if (!p) return fail(MK_E_INVALID, "null plan");
  if (p->graph_only) return fail(MK_E_STATE, "graph-only plans cannot run");
  hipStream_t s = (hipStream_t)stream;
  mk_status st = refuse_capture(s, "mk_run");
  if (st != MK_OK) return st;
  st = ensure_device(p);
  if (st != MK_OK) return st;
  st = bind_operands(p, w, kv_cache, tokens, s, own_bind(p));
  if (st != MK_OK) return st;
  return launch_step(p, s);
}

static mk_status launch_step(mk_plan* p, hipStream_t s) {
  // counters restart from zero after a failed run (some events stopped short of
  // their targets) and before the epoch would wrap to 0, which marks "no error"
  // in the watchdog record
  if (p->need_reset || p->epoch == 0xFFFFFFFFu) {
    HIPCHK(hipMemsetAsync(p->d_counters, 0, counter_bytes(p), s), "reset counters");
    p->epoch = 0;
    p->need_reset = false;
  }
  p->epoch += 1;
  p->run_seq += 1;
  if (p->trace_on) HIPCHK(hipMemsetAsync(p->d_trace, 0, (size_t)p->num_cus * p->P.max_len * mkd::kTraceWords * 8, s), "clear trace");
  HIPCHK(mk::launch_megakernel(kargs(p), p->num_cus, s), "megakernel launch");
  return MK_OK;
}

mk_status mk_run_layerwise(mk_plan* p, const mk_weights* w, void* kv_cache, const void* tokens, void* stream) {
  g_err.clear();
  if (!p) return fail(MK_E_INVALID, "null plan");
  if (p->graph_only) return fail(MK_E_STATE, "graph-only plans cannot run");
  hipStream_t s = (hipStream_t)stream;
  mk_status st = ensure_device(p);
  if (st != MK_OK) return st;
  st = bind_operands(p, w, kv_cache, tokens, s, own_bind(p));
  if (st != MK_OK) return st;
  return launch_layerwise(p, s);
}

static mk_status launch_layerwise(mk_plan* p, hipStream_t s) {
  p->run_seq += 1;
  mkd::KArgs a = kargs(p);
  a.trace = nullptr;
  if (p->n_streams == 1) {
    for (size_t o = 0; o < p->ops.size(); ++o)
      HIPCHK(mk::launch_layer(a, p->num_cus, p->op_first[o], p->op_count[o], s), "layer launch");
    return MK_OK;
  }
  // branches on streams of their own: fork from the caller's stream, wait on
  // each producer launched elsewhere, join every stream back at the end (the
  // same pattern is valid under stream capture)
  if (p->xs.empty()) {
    p->xs.assign(p->n_streams, nullptr);
    for (int k = 1; k < p->n_streams; ++k) HIPCHK(hipStreamCreateWithFlags(&p->xs[k], hipStreamNonBlocking), "stream");
    p->op_done.assign(p->ops.size(), nullptr);
    for (auto& e : p->op_done) HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming), "event");
    HIPCHK(hipEventCreateWithFlags(&p->ev_fork, hipEventDisableTiming), "event");
  }
  auto stream_of = [&](int k) { return k == 0 ? s : p->xs[k]; };
  HIPCHK(hipEventRecord(p->ev_fork, s), "fork");
  for (int k = 1; k < p->n_streams; ++k) HIPCHK(hipStreamWaitEvent(p->xs[k], p->ev_fork, 0), "fork wait");
  std::vector<int> tail(p->n_streams, -1);
  for (size_t o = 0; o < p->ops.size(); ++o) {
    const int k = p->op_stream[o];
    hipStream_t so = stream_of(k);
    for (int q : p->op_prod[o])
      if (p->op_stream[q] != k) HIPCHK(hipStreamWaitEvent(so, p->op_done[q], 0), "wait producer");
    HIPCHK(mk::launch_layer(a, p->num_cus, p->op_first[o], p->op_count[o], so), "layer launch");
    HIPCHK(hipEventRecord(p->op_done[o], so), "op done");
    tail[k] = (int)o;
  }
  for (int k = 1; k < p->n_streams; ++k)
    if (tail[k] >= 0) HIPCHK(hipStreamWaitEvent(s, p->op_done[tail[k]], 0), "join");
  return MK_OK;
}

// ---- new sequence lengths without replanning; runs of steps -------------------
// A step at lengths kv differs from the planned one only in the attention
// tasks' payloads (split ranges and position) and the RoPE table: the queue's
// shape, events and targets do not depend on the lengths.
static mk_status check_lengths(const mk_plan* p, const std::vector<int32_t>& kv) {
  if (p->graph_only) return fail(MK_E_STATE, "graph-only plans have no sequence lengths");
  if (p->glm) return fail(MK_E_UNSUPPORTED, "the GLM path's token positions are fixed by its plan");
  const mk_model_desc& d = p->desc;
  int maxpos = 0;
  for (int b = 0; b < p->batch; ++b) {
    if (kv[b] < 0 || kv[b] + 1 > d.max_kv_len) return fail(MK_E_UNSUPPORTED, "kv_len[b] + 1 must be <= max_kv_len");
    maxpos = std::max(maxpos, kv[b] + 1);
  }
  // (batched head_dim-64 attention streams its rows through the ring: any length)
  const long ring = (long)mk::ring_pages(p->batch) * mkd::kPage;
  const long rows = mk::ceil_div(maxpos, p->opts.attn_splits);
  const bool streams = p->batch > 1 && d.head_dim == 64;
  if (!streams && (rows * d.head_dim * 2 + 1023) / 1024 * 1024 * 2 > ring)
    return fail(MK_E_UNSUPPORTED, "an attention split no longer fits the LDS page ring: build a new plan");
  return MK_OK;
}

// Host side: patch the queue copy and the RoPE table for lengths kv; write the
// attention patches (word index, lo, hi, pos) to out (4 int32 each) if given.
static void apply_lengths(mk_plan* p, const std::vector<int32_t>& kv, int32_t* out) {
  p->kv_len = kv;
  p->version += 1;
  const int S = p->opts.attn_splits;
  for (size_t j = 0; j < p->attn_words.size(); ++j) {
    int32_t* w = &p->P.queue[p->attn_words[j]];
    const int b = w[mkd::WGx], sp = w[mkd::WGz], pos = kv[b];
    int lo = 0, hi = 0;
    mk::split_range(pos, S, sp, &lo, &hi);
    w[mkd::WPay] = lo;
    w[mkd::WPay + 1] = hi;
    w[mkd::WPay + 2] = pos;
    if (out) {
      out[4 * j] = p->attn_words[j] + mkd::WPay;
      out[4 * j + 1] = lo;
      out[4 * j + 2] = hi;
      out[4 * j + 3] = pos;
    }
  }
  rope_table(p);
}

// Stage n steps at lengths kv + k (k = 0 .. n-1) in pinned host memory and copy
// them to the device on stream s (*dev: the device copy); the host state ends at
// the last step's lengths.
static mk_status stage_steps(mk_plan* p, const std::vector<int32_t>& kv, int n, hipStream_t s, size_t* step_bytes,
                             const char** dev) {
  const size_t pbytes = p->attn_words.size() * 16, rbytes = p->h_rope.size() * 4;
  const size_t per = (pbytes + rbytes + 255) / 256 * 256;
  *step_bytes = per;
  mk_plan::Staging& g = p->stg[p->stg_next];
  p->stg_next ^= 1;
  if (g.ev) HIPCHK(hipEventSynchronize(g.ev), "earlier staging");  // host buffer reuse
  if ((size_t)n * per > g.cap) {
    // hipFree waits for the device, so no queued set-up kernel still reads g.d
    if (g.h) HIPCHK(hipHostFree(g.h), "hipHostFree");
    if (g.d) HIPCHK(hipFree(g.d), "hipFree");
    g.h = nullptr;
    g.d = nullptr;
    g.cap = 0;
    HIPCHK(hipHostMalloc((void**)&g.h, (size_t)n * per, hipHostMallocDefault), "hipHostMalloc steps");
    HIPCHK(hipMalloc((void**)&g.d, (size_t)n * per), "hipMalloc steps");
    g.cap = (size_t)n * per;
  }
  if (!g.ev) HIPCHK(hipEventCreateWithFlags(&g.ev, hipEventDisableTiming), "event");
  std::vector<int32_t> k_kv(kv);
  for (int k = 0; k < n; ++k) {
    for (int b = 0; b < p->batch; ++b) k_kv[b] = kv[b] + k;
    char* h = g.h + (size_t)k * per;
    apply_lengths(p, k_kv, (int32_t*)h);
    std::memcpy(h + pbytes, p->h_rope.data(), rbytes);
  }
  HIPCHK(hipMemcpyAsync(g.d, g.h, (size_t)n * per, hipMemcpyHostToDevice, s), "upload steps");
  HIPCHK(hipEventRecord(g.ev, s), "staging event");
  *dev = g.d;
  return MK_OK;
}

// Step k of a staged run: patch the queue and install its RoPE table; with
// ntok > 0 also hand the previous step's next tokens to the token buffer (and
// to out, if given) -- one launch.
static mk_status install_step(mk_plan* p, const char* staged, int k, size_t per, hipStream_t s, int ntok = 0,
                              int* out = nullptr) {
  const char* d = staged + (size_t)k * per;
  HIPCHK(mk::launch_step_setup(p->d_queue, d, (int)p->attn_words.size(), p->d_rope,
                               (const float*)(d + p->attn_words.size() * 16), (int)p->h_rope.size(), p->d_tok,
                               (const int*)(p->d_ws + p->off_next), out, ntok, s),
         "step set-up");
  return MK_OK;
}

mk_status mk_plan_set_kv_len(mk_plan* p, const int32_t* kv_len, void* stream) {
  g_err.clear();
  if (!p || !kv_len) return fail(MK_E_INVALID, "null argument");
  std::vector<int32_t> kv(kv_len, kv_len + std::max(0, p->batch));
  mk_status st = check_lengths(p, kv);
  if (st != MK_OK) return st;
  if (!p->uploaded) {  // the first run uploads the patched queue and table
    apply_lengths(p, kv, nullptr);
    return MK_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  size_t per = 0;
  const char* staged = nullptr;
  st = stage_steps(p, kv, 1, s, &per, &staged);
  if (st != MK_OK) return st;
  return install_step(p, staged, 0, per, s);
}

mk_status mk_run_steps(mk_plan* p, const mk_weights* w, void* kv_cache, const void* tokens, int32_t n_steps,
                       void* out_tokens, int32_t layerwise, void* stream) {
  g_err.clear();
  if (!p) return fail(MK_E_INVALID, "null plan");
  if (n_steps < 1) return fail(MK_E_INVALID, "n_steps must be >= 1");
  std::vector<int32_t> last(p->kv_len);
  for (auto& v : last) v += n_steps - 1;
  mk_status st = check_lengths(p, last);
  if (st != MK_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = refuse_capture(s, "mk_run_steps");
  if (st != MK_OK) return st;
  st = ensure_device(p);
  if (st != MK_OK) return st;
  if (!p->d_tok) HIPCHK(hipMalloc((void**)&p->d_tok, (size_t)p->batch * 4), "hipMalloc tokens");
  if (!tokens) return fail(MK_E_INVALID, "null token pointer");
  HIPCHK(hipMemcpyAsync(p->d_tok, tokens, (size_t)p->batch * 4, hipMemcpyDeviceToDevice, s), "first tokens");
  st = bind_operands(p, w, kv_cache, p->d_tok, s, own_bind(p));
  if (st != MK_OK) return st;
  const std::vector<int32_t> first(p->kv_len);
  size_t per = 0;
  const char* staged = nullptr;
  st = stage_steps(p, first, n_steps, s, &per, &staged);
  if (st != MK_OK) return st;
  const char* next = p->d_ws + p->off_next;
  for (int k = 0; k < n_steps; ++k) {
    if (k > 0) {  // step k's lengths and RoPE; step k - 1's next tokens in, and out
      int* out = out_tokens ? (int*)out_tokens + (size_t)(k - 1) * p->batch : nullptr;
      st = install_step(p, staged, k, per, s, p->batch, out);
      if (st != MK_OK) return st;
    }
    st = layerwise ? launch_layerwise(p, s) : launch_step(p, s);
    if (st != MK_OK) return st;
  }
  if (out_tokens)
    HIPCHK(hipMemcpyAsync((char*)out_tokens + (size_t)(n_steps - 1) * p->batch * 4, next, (size_t)p->batch * 4,
                          hipMemcpyDeviceToDevice, s), "copy out tokens");
  return MK_OK;
}


mk_status mk_plan_output(const mk_plan* p, int32_t which, void** dev_ptr, size_t* bytes) {
  g_err.clear();
  if (!p || !dev_ptr || !bytes) return fail(MK_E_INVALID, "null argument");
  if (p->graph_only || !p->uploaded) return fail(MK_E_STATE, "the plan has not run");
  const size_t B = p->batch;
  if (p->glm) {
    const mk_model_desc& d = p->desc;
    const size_t H = d.hidden;
    size_t off = 0, n = 0;
    switch (which) {
      case MK_OUT_GLM_R: off = p->off_gr; n = B * H * 2; break;
      case MK_OUT_GLM_Q: off = p->off_gq; n = B * d.n_q_heads * d.head_dim * 2; break;
      case MK_OUT_GLM_QIDX: off = p->off_gqidx; n = B * d.n_idx_heads * d.idx_head_dim * 2; break;
      case MK_OUT_GLM_GATE: off = p->off_ggate; n = B * d.n_gate * 4; break;
      case MK_OUT_GLM_NORM: off = p->off_gn; n = B * H * 4; break;
      case MK_OUT_GLM_ACT: off = p->off_ga8; n = B * H; break;
      case MK_OUT_GLM_ACT_SCALE: off = p->off_gas; n = B * (H / 128) * 4; break;
      case MK_OUT_GLM_QKVA: off = p->off_gqkva; n = B * (size_t)p->c.na * 4; break;
      case MK_OUT_GLM_QA: off = p->off_gqa8; n = B * d.q_lora; break;
      case MK_OUT_GLM_QA_SCALE: off = p->off_gqs; n = B * (d.q_lora / 128) * 4; break;
      default:
        return fail(MK_E_INVALID, "unknown output for the GLM path");
    }
    *dev_ptr = p->d_ws + off;
    *bytes = n;
    return MK_OK;
  }
  switch (which) {
    case MK_OUT_LOGITS:
      *dev_ptr = p->d_ws + p->off_logits;
      *bytes = B * p->c.V * 4;
      return MK_OK;
    case MK_OUT_NEXT_TOKEN:
      *dev_ptr = p->d_ws + p->off_next;
      *bytes = B * 4;
      return MK_OK;
    case MK_OUT_QKV:
      *dev_ptr = p->d_ws + p->off_qkv;
      *bytes = p->sz_qkv * p->c.L;
      return MK_OK;
    case MK_OUT_HIDDEN:
      *dev_ptr = p->d_ws + p->off_hidden;
      *bytes = p->sz_hid * 2 * p->c.L;
      return MK_OK;
    default:
      return fail(MK_E_INVALID, "unknown output");
  }
}

mk_status mk_plan_copy_output(const mk_plan* p, int32_t which, void* dst, size_t bytes, void* stream) {
  void* src = nullptr;
  size_t n = 0;
  mk_status st = mk_plan_output(p, which, &src, &n);
  if (st != MK_OK) return st;
  if (!dst || bytes < n) return fail(MK_E_INVALID, "destination missing or too small");
  HIPCHK(hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, (hipStream_t)stream), "copy output");
  return MK_OK;
}

mk_status mk_plan_check(mk_plan* p, void* stream, mk_check* out) {
  g_err.clear();
  if (!p || !out) return fail(MK_E_INVALID, "null argument");
  std::memset(out, 0, sizeof(*out));
  if (p->graph_only || !p->uploaded) return fail(MK_E_STATE, "the plan has not run");
  HIPCHK(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  std::vector<uint32_t> ctr(counter_bytes(p) / 4);
  uint32_t err[16];
  HIPCHK(hipMemcpy(ctr.data(), p->d_counters, ctr.size() * 4, hipMemcpyDeviceToHost), "read counters");
  HIPCHK(hipMemcpy(err, p->d_err, 64, hipMemcpyDeviceToHost), "read err");
  out->epoch = p->epoch;
  int bad = 0;
  for (int e = 0; e < p->P.num_events; ++e) {
    uint32_t sum = 0;  // modulo 2^32, as the device compares
    for (int k = 0; k < mkd::kCtrSub; ++k) sum += ctr[mkd::ctr_word(e, k, p->P.num_events)];
    if (sum != p->epoch * p->P.event_target[e]) ++bad;
  }
  out->bad_counters = bad;
  out->counters_ok = bad == 0;
  if (err[0] != 0 && err[0] == p->epoch) {
    out->err_kind = (int32_t)err[1];
    out->err_cu = (int32_t)err[2];
    out->err_slot = (int32_t)err[3];
    out->err_event = (int32_t)err[4];
    out->err_value = err[5];
    out->err_target = err[6];
    p->need_reset = true;
    return fail(MK_E_TIMEOUT, "a device wait timed out (kind " + std::to_string(err[1]) + ", cu " + std::to_string(err[2]) +
                                  ", slot " + std::to_string(err[3]) + ")");
  }
  if (bad) p->need_reset = true;
  if (p->run_seq != 0 && err[7] == p->run_seq)
    return fail(MK_E_INVALID, "an input token id was outside [0, vocab) (the step ran on the clamped id)");
  return MK_OK;
}

mk_status mk_plan_set_trace(mk_plan* p, int32_t enable) {
  g_err.clear();
  if (!p) return fail(MK_E_INVALID, "null plan");
  if (p->graph_only) return fail(MK_E_STATE, "graph-only plans cannot run");
  if (enable && !p->d_trace) {
    HIPCHK(hipMalloc(&p->d_trace, (size_t)p->num_cus * p->P.max_len * mkd::kTraceWords * 8), "hipMalloc trace");
  }
  p->trace_on = enable != 0;
  return MK_OK;
}

mk_status mk_plan_trace(mk_plan* p, void* stream, uint64_t* host_out, size_t bytes, double* ticks_per_us) {
  g_err.clear();
  if (!p || !host_out || !ticks_per_us) return fail(MK_E_INVALID, "null argument");
  const size_t need = (size_t)p->num_cus * p->P.max_len * mkd::kTraceWords * 8;
  if (!p->d_trace) return fail(MK_E_STATE, "tracing was never enabled");
  if (bytes < need) return fail(MK_E_INVALID, "host buffer too small");
  HIPCHK(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize");
  HIPCHK(hipMemcpy(host_out, p->d_trace, need, hipMemcpyDeviceToHost), "read trace");
  *ticks_per_us = p->ticks_per_us;
  return MK_OK;
}

// ---- the allocation-free entry point -----------------------------------------
// Per device: the address of the static buffer, and which plan state it holds.
namespace {
constexpr int kMaxDevices = 64;
struct ScratchDev {
  void* base = nullptr;                 // device address of 'scratch' on this device
  uint64_t owner_uid = 0, owner_ver = 0;  // plan whose queue and RoPE table it holds
  std::vector<uint64_t> optab;          // host copy of its operand table
};
std::mutex g_scratch_mu;
ScratchDev g_scratch[kMaxDevices];

size_t r256(size_t v) { return (v + 255) / 256 * 256; }

// The buffer's layout for plan p: queue, counters, watchdog record, operand
// table, RoPE table, then the workspace up to (not including) the outputs.
struct ScratchLayout {
  size_t queue, counters, err, optab, rope, ws, total;
};
ScratchLayout scratch_layout(const mk_plan* p) {
  ScratchLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += r256(bytes);
    return o;
  };
  l.queue = take(p->P.queue.size() * 4);
  l.counters = take((size_t)mkd::kCtrSub * std::max(1, p->P.num_events) * mkd::kCtrStride * 4);
  l.err = take(64);
  l.optab = take(p->ops.size() * 16 * 8);
  l.rope = take((size_t)p->batch * p->c.hd * 4);
  l.ws = take(p->off_logits);
  l.total = off;
  return l;
}
}  // namespace

mk_status mk_run_noalloc(mk_plan* p, const mk_weights* w, void* kv_cache, const void* tokens, void* logits,
                         void* next_tokens, void* stream) {
  g_err.clear();
  if (!p || !logits || !next_tokens) return fail(MK_E_INVALID, "null plan or output pointer");
  if (p->graph_only) return fail(MK_E_STATE, "graph-only plans cannot run");
  if (p->glm) return fail(MK_E_UNSUPPORTED, "mk_run_noalloc runs Llama-family plans only");
  hipStream_t s = (hipStream_t)stream;
  mk_status st = refuse_capture(s, "mk_run_noalloc");
  if (st != MK_OK) return st;
  int dev = -1;
  HIPCHK(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MK_E_UNSUPPORTED, "device index out of range");
  const ScratchLayout lay = scratch_layout(p);
  if (lay.total > kScratchBytes)
    return fail(MK_E_UNSUPPORTED, "the plan needs " + std::to_string(lay.total) + " bytes of device scratch; mk_run_noalloc "
                                  "holds at most " + std::to_string(kScratchBytes) + " (use mk_run)");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  ScratchDev& sd = g_scratch[dev];
  if (!sd.base) {
    // once per device, with that device current
    void* ptr = nullptr;
    HIPCHK(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(MK_E_HIP, "hipGetSymbolAddress(scratch) returned null");
    sd.base = ptr;
  }
  // the grid must be co-resident (queries only, no allocation)
  int ncu = 0, occ = 0;
  HIPCHK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev), "hipDeviceGetAttribute");
  HIPCHK(mk::megakernel_occupancy(p->c.hd, p->batch, false, &occ), "occupancy");
  if (p->num_cus > ncu || occ < 1) return fail(MK_E_UNSUPPORTED, "the persistent grid cannot be co-resident");
  int clk_khz = 0;
  HIPCHK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeWallClockRate, dev), "hipDeviceGetAttribute clock");
  if (clk_khz <= 0) return fail(MK_E_HIP, "the device reports no constant clock rate");
  char* base = (char*)sd.base;
  int* queue = (int*)(base + lay.queue);
  unsigned* counters = (unsigned*)(base + lay.counters);
  unsigned* err = (unsigned*)(base + lay.err);
  uint64_t* optab = (uint64_t*)(base + lay.optab);
  float* rope = (float*)(base + lay.rope);
  char* ws = base + lay.ws;
  // the buffer keeps the last call's contents: the queue and RoPE table are
  // copied in when another plan (or another state of this one) used it last
  if (sd.owner_uid != p->uid || sd.owner_ver != p->version) {
    if (p->h_rope.empty()) rope_table(p);
    HIPCHK(hipMemcpyAsync(queue, p->P.queue.data(), p->P.queue.size() * 4, hipMemcpyHostToDevice, s), "upload queue");
    HIPCHK(hipMemcpyAsync(rope, p->h_rope.data(), p->h_rope.size() * 4, hipMemcpyHostToDevice, s), "upload rope");
    sd.optab.clear();  // the table sits elsewhere in the new layout
    sd.owner_uid = p->uid;
    sd.owner_ver = p->version;
  }
  Bind b{ws, rope, (float*)logits, (int*)next_tokens, optab, &sd.optab};
  st = bind_operands(p, w, kv_cache, tokens, s, b);
  if (st != MK_OK) return st;
  // every call starts its counters and watchdog record from zero, at epoch 1
  HIPCHK(hipMemsetAsync(counters, 0, (size_t)mkd::kCtrSub * std::max(1, p->P.num_events) * mkd::kCtrStride * 4, s),
         "clear counters");
  HIPCHK(hipMemsetAsync(err, 0, 64, s), "clear watchdog record");
  mkd::KArgs a = kargs(p, queue, optab, counters, err);
  a.epoch = 1;
  a.run_id = 1;
  a.trace = nullptr;
  a.timeout_ticks = (unsigned long long)p->timeout_ms * (unsigned long long)clk_khz;
  HIPCHK(mk::launch_megakernel(a, p->num_cus, s), "megakernel launch");
  return MK_OK;
}

mk_status mk_plan_poison_workspace(mk_plan* p, void* stream) {
  g_err.clear();
  if (!p) return fail(MK_E_INVALID, "null plan");
  if (p->graph_only || !p->uploaded) return fail(MK_E_STATE, "the plan has not run");
  HIPCHK(hipMemsetAsync(p->d_ws, 0xFF, p->ws_bytes, (hipStream_t)stream), "poison workspace");
  return MK_OK;
}

mk_status mk_plan_debug_raise_wait(mk_plan* p, int32_t event, int32_t delta, int32_t slot) {
  g_err.clear();
  if (!p) return fail(MK_E_INVALID, "null plan");
  if (p->graph_only) return fail(MK_E_STATE, "graph-only plans cannot run");
  if (event < 0 || event >= p->P.num_events) return fail(MK_E_INVALID, "event out of range");
  if (slot < 0 || slot > 2) return fail(MK_E_INVALID, "slot must be 0, 1 or 2");
  for (size_t t = 0; t * 32 < p->P.queue.size(); ++t) {
    int32_t* w = &p->P.queue[t * 32];
    if (w[mkd::WOpcode] == mkd::OpNoop) continue;
    if (slot != 2 && w[mkd::WWaitCnt] >= 1 && w[mkd::WWaitEv] == event) w[mkd::WWaitTgt] += delta;
    if (slot != 1 && w[mkd::WWaitCnt] == 2 && w[mkd::WWait2Ev] == event) w[mkd::WWait2Tgt] += delta;
  }
  p->version += 1;
  if (p->uploaded)
    HIPCHK(hipMemcpy(p->d_queue, p->P.queue.data(), p->P.queue.size() * 4, hipMemcpyHostToDevice), "upload queue");
  return MK_OK;
}

mk_status mk_stream_probe(const void* src, size_t bytes, int32_t lds_dma, int32_t workgroups, int32_t waves,
                          int32_t depth, void* sink, void* stream) {
  g_err.clear();
  if (!src || !sink) return fail(MK_E_INVALID, "null buffer");
  if (bytes == 0 || bytes % mkd::kPage) return fail(MK_E_INVALID, "bytes must be a positive multiple of 16 KiB");
  if (workgroups < 1 || waves < 1 || waves > 8 || depth < 1 || depth > (lds_dma ? 4 : 2))
    return fail(MK_E_INVALID, "workgroups >= 1, waves 1..8, depth 1..4 (LDS-DMA) or 1..2 (register loads)");
  HIPCHK(mk::launch_stream_probe(src, (long)(bytes / mkd::kPage), lds_dma, workgroups, waves, depth, (unsigned*)sink,
                                 (hipStream_t)stream),
         "stream probe launch");
  return MK_OK;
}

mk_status mk_noalloc_bytes(const mk_plan* p, size_t* need, size_t* limit) {
  g_err.clear();
  if (!p || !need || !limit) return fail(MK_E_INVALID, "null argument");
  *need = (p->graph_only || p->glm) ? 0 : scratch_layout(p).total;
  *limit = kScratchBytes;
  return MK_OK;
}

void mk_plan_free(mk_plan* p) {
  if (!p) return;
  if (p->uploaded) {
    (void)hipDeviceSynchronize();
    (void)hipFree(p->d_queue);
    (void)hipFree(p->d_counters);
    (void)hipFree(p->d_err);
    (void)hipFree(p->d_optab);
    (void)hipFree(p->d_rope);
    (void)hipFree(p->d_ws);
    if (p->d_rows) (void)hipFree(p->d_rows);
    if (p->d_patch) (void)hipFree(p->d_patch);
    for (auto& g : p->stg)
      if (g.d) (void)hipFree(g.d);
    if (p->d_tok) (void)hipFree(p->d_tok);
  }
  if (p->d_trace) (void)hipFree(p->d_trace);
  for (size_t k = 1; k < p->xs.size(); ++k)
    if (p->xs[k]) (void)hipStreamDestroy(p->xs[k]);
  for (auto e : p->op_done)
    if (e) (void)hipEventDestroy(e);
  if (p->ev_fork) (void)hipEventDestroy(p->ev_fork);
  for (auto& g : p->stg) {
    if (g.ev) (void)hipEventDestroy(g.ev);
    if (g.h) (void)hipHostFree(g.h);
  }
  delete p;
}

}  // extern "C"
