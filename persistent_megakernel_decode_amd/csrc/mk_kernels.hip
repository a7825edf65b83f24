// Persistent megakernel interpreter and layerwise kernels for gfx950 (MI355X).
//
// Megakernel: one workgroup per compute unit walks its static queue of tile
// instructions.  The worker loop is the one of the CMU 15-779 lecture 7 notes,
// section 4.1 (fetch the task, prefetch its weights without waiting on any
// dependency, wait for the counters, read activations and compute, bump the
// trigger counter), split over wavefront roles as in the MegaRTP article,
// section 3 (controller / loader / consumer / storer warps) and section 4
// ("Device-side execution", "shared-memory paging"):
//   wave 0    controller: stages each instruction's record in LDS, waits
//             for its event counter and publishes "ready" in LDS (the reads
//             that follow need no acquire: see CohT in mk_device.hpp);
//   wave 1    storer: after the compute waves finish an instruction, runs
//             the epilogue, waits for the outputs' stores to complete and
//             adds to the trigger counter (relaxed, agent scope);
//   waves 2-3 weight loaders: stream every instruction's weight (or K/V) bytes
//             HBM -> LDS with LDS-DMA (global_load_lds_dwordx4), alternating
//             16 KiB pages of a 9-page ring; they never wait on events, only on
//             free pages, so weights stream while activations are not ready;
//   waves 4-7 compute: one quarter of K each (GEMV) or one query head each
//             (attention); the last of them to finish runs the epilogue.
// Every wait is bounded (watchdog): on timeout the wave records
// {cu, slot, event, value, target} and the workgroup drains and exits.
#include <hip/hip_runtime.h>

#include "mk_device.hpp"
#include "mk_glm.hpp"

using namespace mkd;

namespace {

typedef __attribute__((address_space(3))) void lds_void;

// PW / SW: partial-sum and sum-of-squares floats per compute wave per slot
// (one value per tile row for batch 1; a 16 x 16 block of rows x sequences and
// one value per sequence for the batched path); NWT: compute waves in all
template <int PW, int SW, int NWT>
struct CtrlT {
  int ready_seq, done_seq, abort_flag, meta_seq;  // meta_seq: meta records staged (instructions 0 .. meta_seq-1)
  int slot_full[16];   // generation + 1 of the data in each ring slot (loaders -> compute)
  int slot_rel[16];    // compute-wave releases of each slot, cumulative (kNW per use)
  int arrive[4];       // compute waves done with instruction i (slot i % 4)
  int xch[4];          // compute waves that posted a partial sum for instruction i (slot i % 4)
  int rel_sink[64];    // target of the zero adds of lanes that release no page
  float part[4][kNW][PW];
  float ssp[4][kNW][SW];
  float scratch[NWT][kScratch];
};
// Copies of the instructions in flight (instruction i in slot i % kMeta) and of
// their operand-table rows, staged by the controller.
constexpr int kMeta = 8;
// Workgroup LDS.  MB: batched sequences (MFMA tiles) -- one page less in the
// ring for the 16 x 16 partial blocks.  SETS: groups of kNW compute waves; with
// two, consecutive instructions alternate between the groups, so that one
// tile's activation loads and matrix-core work overlap the next one's (the
// batched path: its tiles are bound by the latency of those loads, and its
// registers leave room for a third wave per SIMD).
template <bool MB_, bool GLM_ = false>
struct __attribute__((aligned(16))) LdsT {
  static constexpr bool MB = MB_;
  static constexpr bool GLM = GLM_;  // the GLM pre-attention interpreter (batched layout)
  static constexpr int NP = MB_ ? kNumPages - 1 : kNumPages;  // ring pages
  static constexpr int PW = MB_ ? kMB * kMB : kMaxRows;
  static constexpr int SW = MB_ ? kMB : 1;
  static constexpr int SETS = (MB_ && !GLM_) ? 2 : 1;
  static constexpr int THREADS = (4 + kNW * SETS) * 64;
  char ring[NP][kPage];
  uint32_t meta[kMeta][64];
  CtrlT<PW, SW, kNW * SETS> c;
};
static_assert(sizeof(LdsT<true>) <= 160 * 1024 && sizeof(LdsT<false>) <= 160 * 1024 &&
                  sizeof(LdsT<true, true>) <= 160 * 1024,
              "workgroup LDS above 160 KiB");

template <class T>
__device__ __forceinline__ uint32_t lds_addr(LDS T* p) {
  return (uint32_t)(uintptr_t)p;
}
// LDS flag access for the loader waves, in inline asm so that the compiler
// does not put a vmcnt(0) wait (for the wave's own pending LDS-DMA) in front.
__device__ __forceinline__ int lds_ld_asm(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void lds_st_asm(uint32_t addr, int v) {
  asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ int lds_load_acq(LDS int* p) { return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP); }
// Publish an LDS flag: orders the wave's earlier LDS accesses only (a release
// over all address spaces would also wait for the wave's global stores).
__device__ __forceinline__ void lds_store_rel(LDS int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP); }

enum { ErrEvent = 1, ErrPage = 2, ErrReady = 3, ErrDrain = 4, ErrFree = 5 };

// The record belongs to the run whose epoch is in err[0]; the first failing
// wave of that run fills it.
template <class LT>
__device__ void record_error(const KArgs& a, LDS LT* L, int kind, int slot, int ev, unsigned val, unsigned tgt) {
  if (lane_id() == 0) {
    unsigned old = __hip_atomic_load(&a.err[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old != a.epoch && __hip_atomic_compare_exchange_strong(&a.err[0], &old, a.epoch, __ATOMIC_RELAXED,
                                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
      a.err[1] = kind;
      a.err[2] = blockIdx.x;
      a.err[3] = slot;
      a.err[4] = ev;
      a.err[5] = val;
      a.err[6] = tgt;
    }
    __hip_atomic_store(&L->c.abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

template <class LT>
__device__ __forceinline__ bool aborted(LDS LT* L) {
  return __hip_atomic_load(&L->c.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
}

// Wait until *p >= v (LDS, workgroup acquire), bounded.
template <class LT>
__device__ bool wait_lds_ge(const KArgs& a, LDS LT* L, LDS int* p, int v, int kind, int slot) {
  if (lds_load_acq(p) >= v) return true;
  const unsigned long long t0 = now_ticks();
  for (unsigned it = 0;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    if (lds_load_acq(p) >= v) return true;
    if ((it & 31) == 31) {
      if (aborted(L)) return false;
      if (now_ticks() - t0 > a.timeout_ticks) {
        record_error(a, L, kind, slot, -1, (unsigned)lds_load_acq(p), (unsigned)v);
        return false;
      }
    }
  }
}

// Input token ids outside [0, vocab): the tiles read a clamped id (no access
// leaves the embedding), and the run is flagged in err[7] (= the run's id), so
// that mk_plan_check reports it.  Done by the layer-0 QKV tiles, which are the
// first to read the tokens.
__device__ __forceinline__ void check_tokens(const KArgs& a, const Meta& m) {
  if (m.w(WOpcode) != OpQkv || m.w(WLayer) != 0 || m.q(QkvX) != 0) return;
  const int lane = lane_id();
  const int t = lane < a.c.B ? ((const GLB int*)m.q(QkvTokens))[lane] : 0;
  if (t < 0 || t >= a.c.V) __hip_atomic_store(&a.err[7], a.run_id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ const CST int* instr(const KArgs& a, int i) {
  return (const CST int*)(uintptr_t)a.queue + ((size_t)blockIdx.x * a.max_len + i) * 32;
}
__device__ __forceinline__ const CST uint64_t* oprow(const KArgs& a, int row) {
  return (const CST uint64_t*)(uintptr_t)a.optab + (size_t)row * 16;
}

// Copy instruction j and its operand row into meta record j % kMeta (scalar
// loads; lane 0 writes).  With two compute groups the record also carries the
// sequence number of the instruction's first ring page (pages: pages of
// instructions 0 .. j-1; instructions are staged in order); a single group
// counts them itself.  Past the end of the queue the record is a NoOp.
template <class LT>
__device__ void stage(const KArgs& a, LDS LT* L, int j, int& pages) {
  LDS uint32_t* rec = L->meta[j % kMeta];
  if (j >= a.max_len) {
    if (lane_id() == 0) rec[WOpcode] = OpNoop;
    return;
  }
  const CST uint32_t* g = (const CST uint32_t*)instr(a, j);
  uint32_t w[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) w[k] = g[k];
  if (lane_id() == 0) {
#pragma unroll
    for (int k = 0; k < 32; ++k) rec[k] = k == WFirstPage ? (uint32_t)pages : w[k];
  }
  if (LT::SETS > 1 && (int)w[WOpcode] != OpNoop) {
    GMeta gm;
    gm.ins = (const CST int*)g;
    gm.row = oprow(a, (int)w[WOpRow]);
    pages += tile_info(gm, a.c).npages;
  }
  const CST uint32_t* gr = (const CST uint32_t*)oprow(a, (int)w[WOpRow]);
#pragma unroll
  for (int k = 0; k < 32; ++k) w[k] = gr[k];
  if (lane_id() == 0) {
#pragma unroll
    for (int k = 0; k < 32; ++k) rec[32 + k] = w[k];
  }
}

// ---------------------------------------------------------------------------
template <class LT>
__device__ __forceinline__ void controller(const KArgs& a, LDS LT* L) {
  // per wait slot, the last event this wave saw at or past a target and the
  // count it read: counters only grow within a run, so a later instruction
  // waiting on the same event for a target within that count needs neither a
  // poll nor an acquire
  int seen_ev[2] = {-1, -1};
  unsigned seen_val[2] = {0u, 0u};
  int pages = 0;
  stage(a, L, 0, pages);
  if (lane_id() == 0) lds_store_rel(&L->c.meta_seq, 1);
  for (int i = 0; i < a.max_len; ++i) {
    const Meta m = load_meta(L->meta[i % kMeta]);
    if (m.w(WOpcode) == OpNoop) {
      // let the other waves read the NoOp and leave their loops; with two
      // compute groups the one whose next instruction is i + 1 reads that (a
      // NoOp too: a queue ends at its first NoOp)
      if (LT::SETS > 1) {
        if (i + 2 > kMeta && !wait_lds_ge(a, L, &L->c.done_seq, i + 2 - kMeta, ErrDrain, i)) return;
        stage(a, L, i + 1, pages);
        if (lane_id() == 0) lds_store_rel(&L->c.meta_seq, i + 2);
      }
      if (lane_id() == 0) lds_store_rel(&L->c.ready_seq, i + 1);
      break;
    }
    // slot (i + 1) % kMeta last held instruction i + 1 - kMeta; the storer reads
    // the slots of the instruction it is on and of the next one
    if (i + 2 > kMeta && !wait_lds_ge(a, L, &L->c.done_seq, i + 2 - kMeta, ErrDrain, i)) return;
    stage(a, L, i + 1, pages);
    if (lane_id() == 0) lds_store_rel(&L->c.meta_seq, i + 2);
    // one or two waits (a join waits on both of its producers' events)
    const int nwait = m.w(WWaitCnt);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k >= nwait) break;
      const int ev = m.w(k ? WWait2Ev : WWaitEv);
      const unsigned tgt = a.epoch * (unsigned)m.w(k ? WWait2Tgt : WWaitTgt);
      if ((ev == seen_ev[0] && (int)(seen_val[0] - tgt) >= 0) || (ev == seen_ev[1] && (int)(seen_val[1] - tgt) >= 0))
        continue;
      // lane l reads sub-counters l, l + 64, ... (below kCtrSub); the event's
      // count is their sum
      const int lane = lane_id();
      const int kk = lane < kCtrSub ? lane : 0;
      unsigned* ctr = a.counters + ctr_word(ev, kk, a.num_events);
      const size_t step = ctr_word(0, 64, a.num_events);  // words from sub-counter k to k + 64
      auto count = [&]() {
        unsigned x[kCtrPer];
#pragma unroll
        for (int j = 0; j < kCtrPer; ++j) x[j] = __hip_atomic_load(ctr + j * step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned sum = 0;
#pragma unroll
        for (int j = 0; j < kCtrPer; ++j) sum += x[j];
        return ctr_sum_u32(lane < kCtrSub ? sum : 0u);
      };
      unsigned v = count();
      if ((int)(v - tgt) < 0) {
        const unsigned long long t0 = now_ticks();
        for (unsigned it = 0;; ++it) {
          v = count();  // each poll is a memory round trip: no sleep between them
          if ((int)(v - tgt) >= 0) break;
          if ((it & 15) == 15) {
            if (aborted(L) || __hip_atomic_load(&a.err[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.epoch) {
              if (lane_id() == 0) __hip_atomic_store(&L->c.abort_flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
              return;
            }
            if (now_ticks() - t0 > a.timeout_ticks) {
              record_error(a, L, ErrEvent, i, ev, v, tgt);
              return;
            }
          }
        }
      }
      // no agent-scope acquire (an L2 invalidate) here: see CohT for why the
      // reads that follow need none
      seen_ev[k] = ev;
      seen_val[k] = v;
    }
    if (a.trace && lane_id() == 0) a.trace[((size_t)blockIdx.x * a.max_len + i) * kTraceWords + 0] = now_ticks();
    if (lane_id() == 0) lds_store_rel(&L->c.ready_seq, i + 1);
  }
}

// ---------------------------------------------------------------------------
// Storer: per instruction, prefetch the residual, wait until every compute wave
// has arrived, run the GEMV epilogue (reduce the partials in LDS, RMSNorm
// scale, residual / SiLU, store), hand the LDS slot back, and signal.  A run of
// consecutive instructions that trigger the same event is signalled once, at
// its end, with the summed increment: a producer never depends on its own
// trigger event, so deferring within the run cannot delay the event.
template <class LT>
__device__ __forceinline__ void storer(const KArgs& a, LDS LT* L) {
  const int lane = lane_id();
  unsigned pending = 0;
  int ss_row = -1;     // batched: operand row whose sums of squares ss_val holds
  float ss_val = 0.f;
  for (int i = 0; i < a.max_len; ++i) {
    // the residual may be read only once the instruction's event has been
    // acquired (the controller publishes "ready" after its acquire)
    if (!wait_lds_ge(a, L, &L->c.ready_seq, i + 1, ErrReady, i)) return;
    const Meta m = load_meta(L->meta[i % kMeta]);
    const int op = m.w(WOpcode);
    if (op == OpNoop) break;
    const int sl = i & 3;
    const bool gemv = is_gemv(op);
    if constexpr (!LT::GLM) check_tokens(a, m);
    if constexpr (LT::GLM) {
      if (!wait_lds_ge(a, L, &L->c.arrive[sl], kNW, ErrDrain, i)) return;
      if (glm_is_gemm(op)) glm_epilogue(m, a.c, &L->c.part[sl][0][0]);
    } else if constexpr (LT::MB) {
      ResMB res = gemv_residual_mb(m, a.c);
      // take the residual into registers here: left pending, its load would
      // make the compiler wait for all of this wave's memory operations
      // (earlier tiles' stores included) wherever those registers are reused
      asm volatile("" : "+v"(res.r0), "+v"(res.r1));
      // the fused norm's sum of squares: the same for every tile of an op
      // (consecutive tiles of the LM head, gate/up, ... reuse it)
      if (gemv) {
        if (m.w(WOpRow) != ss_row) {
          ss_val = gemv_sumsq_mb(m, a.c);
          ss_row = m.w(WOpRow);
        }
        res.ss = ss_val;
      }
      // a K-halved tile is complete once both groups have arrived
      const int arrivals = (LT::SETS > 1 && gemv_k_halves(op, a.c)) ? 2 * kNW : kNW;
      if (!wait_lds_ge(a, L, &L->c.arrive[sl], arrivals, ErrDrain, i)) return;
      if (gemv)
        gemv_epilogue_mb(m, a.c, &L->c.part[sl][0][0], &L->c.ssp[sl][0][0], res);
      else if (op == OpArgmax)
        argmax_final(m, &L->c.part[sl][0][0], LT::PW);
    } else {
      float res = (op == OpOproj || op == OpDown) ? gemv_residual(m, a.c) : 0.f;
      asm volatile("" : "+v"(res));  // in registers now (see the batched branch)
      if (!wait_lds_ge(a, L, &L->c.arrive[sl], kNW, ErrDrain, i)) return;
      if (gemv)
        gemv_epilogue(m, a.c, L->c.part[sl], &L->c.ssp[sl][0][0], res);
      else if (op == OpArgmax)
        argmax_final(m, &L->c.part[sl][0][0], LT::PW);
    }
    if (lane == 0) {
      __hip_atomic_store(&L->c.arrive[sl], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      __hip_atomic_store(&L->c.xch[sl], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      lds_store_rel(&L->c.done_seq, i + 1);
    }
    if (a.trace && lane == 0) a.trace[((size_t)blockIdx.x * a.max_len + i) * kTraceWords + 2] = now_ticks();
    if (m.w(WSigCnt)) {
      pending += (unsigned)m.w(WSigInc);
      // the next instruction was staged before this one was published; runs
      // are merged only between single-signal instructions
      const Meta nx = load_meta(L->meta[(i + 1) % kMeta]);
      const bool same_next = m.w(WSigCnt) == 1 && nx.w(WOpcode) != OpNoop && nx.w(WSigCnt) == 1 &&
                             nx.w(WSigEv) == m.w(WSigEv);
      if (!same_next) {
        // every output of the run was stored agent-coherent, by this wave or by
        // the compute waves, which waited for their stores before arriving:
        // wait for this wave's stores, then count
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0) {
          __hip_atomic_fetch_add(a.counters + ctr_word(m.w(WSigEv), blockIdx.x % kCtrSub, a.num_events), pending,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (m.w(WSigCnt) == 2)
            __hip_atomic_fetch_add(a.counters + ctr_word(m.w(WSig2Ev), blockIdx.x % kCtrSub, a.num_events),
                                   (unsigned)m.w(WSig2Inc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        pending = 0;
      }
    }
    if (a.trace && lane == 0) a.trace[((size_t)blockIdx.x * a.max_len + i) * kTraceWords + 3] = now_ticks();
  }
}

// ---------------------------------------------------------------------------
// Cache policy of the weight DMA: non-temporal (each weight byte is read once
// per step), so the stream does not push the step's activations and partial
// results out of the L2.
constexpr int kDmaNT = 2;

template <class LT>
__device__ __forceinline__ void loader(const KArgs& a, LDS LT* L, int parity) {
  const int lane = lane_id();
  const uint32_t full_base = lds_addr(&L->c.slot_full[0]);
  const uint32_t rel_base = lds_addr(&L->c.slot_rel[0]);
  // issued-but-unpublished pages (oldest first): page sequence number and, for
  // the trace, the instruction whose last page it is (-1 otherwise); scalars,
  // never indexed
  int q0 = 0, q1 = 0, q2 = 0, q3 = 0, l0 = -1, l1 = -1, l2 = -1, l3 = -1, npend = 0;
  auto publish = [&](int sq, int last_of) {
    lds_st_asm(full_base + 4 * (sq % LT::NP), sq / LT::NP + 1);
    if (a.trace && last_of >= 0 && lane == 0)
      a.trace[((size_t)blockIdx.x * a.max_len + last_of) * kTraceWords + 5] = now_ticks();
  };
  auto publish_all = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (npend > 0) publish(q0, l0);
    if (npend > 1) publish(q1, l1);
    if (npend > 2) publish(q2, l2);
    if (npend > 3) publish(q3, l3);
    npend = 0;
  };
  // the batched interpreters keep 8 to 16 KiB in flight per loader wave (their
  // tiles are bound by the latency of activation loads that queue behind the
  // DMA); the batch-1 interpreter keeps dma_pages pages (its larger models are
  // bound by bandwidth)
  constexpr bool half = LT::MB;
  int seq = 0;
  for (int i = 0; i < a.max_len; ++i) {
    const CST int* ins = instr(a, i);
    if (ins[WOpcode] == OpNoop) break;
    GMeta gm;
    gm.ins = ins;
    gm.row = oprow(a, ins[WOpRow]);
    const Tile t = tile_info(gm, a.c);
    const GLB char* dummy = t.len0 > 0 ? t.p0 : t.p1;
    for (int pg = 0; pg < t.npages; ++pg, ++seq) {
      if ((seq & 1) != parity) continue;
      // the slot's previous page (gen uses ago) must have been released by
      // every compute wave
      const int slot = seq % LT::NP, gen = seq / LT::NP;
      if (lds_ld_asm(rel_base + 4 * slot) < kNW * gen) {
        publish_all();
        const unsigned long long t0 = now_ticks();
        for (unsigned it = 0;; ++it) {
          __builtin_amdgcn_s_sleep(1);
          if (lds_ld_asm(rel_base + 4 * slot) >= kNW * gen) break;
          if ((it & 31) == 31) {
            // leave only once this wave's page DMA has landed (the workgroup's
            // LDS must not be written after its waves have ended)
            if (aborted(L)) {
              asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
              return;
            }
            if (now_ticks() - t0 > a.timeout_ticks) {
              record_error(a, L, ErrFree, i, slot, 0, gen);
              asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
              return;
            }
          }
        }
      }
      if (pg == 0 && a.trace && lane == 0) a.trace[((size_t)blockIdx.x * a.max_len + i) * kTraceWords + 4] = now_ticks();
      LDS char* dst = L->ring[slot];
      // a page inside one segment streams from one base address; otherwise each
      // 16-byte chunk picks its segment (chunks past the tile re-read a valid one)
      const int pofs = pg * kPage;
      const GLB char* whole = nullptr;
      if (!t.ilv && pofs + kPage <= t.len0 && !t.stride)
        whole = t.p0 + pofs;
      else if (!t.ilv && t.len1 && pofs >= t.off1 && pofs + kPage <= t.off1 + t.len1)
        whole = t.p1 + (pofs - t.off1);
      // batched interpreters: after each 8 KiB half of a page, wait for the
      // previous half; the wait after a page's first half completes every
      // earlier page (at most one is pending then)
      auto half_wait = [&](int j) {
        if constexpr (half) {
          if (j == 7 || j == 15) {
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            if (j == 7 && npend) {
              publish(q0, l0);
              npend = 0;
            }
          }
        }
      };
      if (whole) {
        const GLB char* src = whole + lane * 16;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          __builtin_amdgcn_global_load_lds((const GLB void*)(src + j * 1024), (lds_void*)(dst + j * 1024), 16, 0, kDmaNT);
          half_wait(j);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int toff = pofs + j * 1024 + lane * 16;
          const GLB char* src = dummy;
          if (t.ilv) {  // chunk toff / 8 KiB: 4 KiB of K rows, then 4 KiB of V rows
            const int o = ((toff >> 13) << 12) + (toff & 4095);
            if (o < t.len0) src = ((toff >> 12) & 1 ? t.p1 : t.p0) + o;
          } else if (toff < t.len0)  // a strided segment's rows are multiples of 16 bytes long
            src = t.stride ? t.p0 + (size_t)(toff / t.seglen) * t.stride + toff % t.seglen : t.p0 + toff;
          else if (toff >= t.off1 && toff < t.off1 + t.len1)
            src = t.p1 + (toff - t.off1);
          __builtin_amdgcn_global_load_lds((const GLB void*)src, (lds_void*)(dst + j * 1024), 16, 0, kDmaNT);
          half_wait(j);
        }
      }
      const int last_of = pg == t.npages - 1 ? i : -1;
      if constexpr (half) {
        q0 = seq;
        l0 = last_of;
        npend = 1;
        continue;
      }
      if (npend == 0) {
        q0 = seq;
        l0 = last_of;
      } else if (npend == 1) {
        q1 = seq;
        l1 = last_of;
      } else if (npend == 2) {
        q2 = seq;
        l2 = last_of;
      } else {
        q3 = seq;
        l3 = last_of;
      }
      ++npend;
      // keep at most 'depth' (1..3) pages in flight: wait for the oldest to
      // land (16 DMA instructions per page; npend == depth + 1 here, so at most
      // four entries q0..q3 are ever held)
      const int depth = a.dma_pages;
      if (npend > depth) {
        if (depth == 1)
          asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else if (depth == 2)
          asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
        publish(q0, l0);
        q0 = q1;
        l0 = l1;
        q1 = q2;
        l1 = l2;
        q2 = q3;
        l2 = l3;
        --npend;
      }
    }
  }
  publish_all();
}

// ---------------------------------------------------------------------------
// Compute waves.  A batch-1 GEMV tile's weights do not depend on any event: as
// soon as the instruction is staged and its pages have landed, each wave reads
// its share into registers and hands the pages back, and only then waits for
// the instruction's event (controller "ready") and loads the activations.
// Other ops wait for "ready" first.
// set: this wave's compute group; group g takes instructions g, g + SETS, ...
// and, with two groups, the second K-half of the other group's K-halved GEMV
// tiles (it reads only these records, each before its arrival, so the
// controller cannot have reused the slot).
template <int HD, class LT>
__device__ __forceinline__ void compute(const KArgs& a, LDS LT* L, int cw, int set) {
  const int lane = lane_id();
  int act_row = -1;
  int seq = 0;  // one group: ring pages of the instructions before i
  Act act;
  for (int i = LT::SETS > 1 ? 0 : set; i < a.max_len; i += LT::SETS > 1 ? 1 : LT::SETS) {
    // two groups: besides its own instructions (i mod 2 = set) a group helps
    // with the other group's K-halved tiles; it tells them from the queue's
    // opcode word (the queue does not change during a run), and reads such a
    // record before arriving on it, so that the slot is still that record's
    bool own = true;
    if constexpr (LT::SETS > 1) {
      own = (i & 1) == set;
      if (!own) {
        const int opg = instr(a, i)[WOpcode];
        if (opg == OpNoop) break;
        if (!gemv_k_halves(opg, a.c)) continue;
      }
    }
    if (!wait_lds_ge(a, L, &L->c.meta_seq, i + 1, ErrReady, i)) return;
    const Meta m = load_meta(L->meta[i % kMeta]);
    const int op = m.w(WOpcode);
    if (op == OpNoop) break;
    const Tile t = tile_info(m, a.c);
    unsigned long long* tr = a.trace ? a.trace + ((size_t)blockIdx.x * a.max_len + i) * kTraceWords : nullptr;
    int first = seq;
    if constexpr (LT::SETS > 1)
      first = m.w(WFirstPage);
    else
      seq += t.npages;
    // the partial-sum slot i % 4 was last used by instruction i - 4
    if (!wait_lds_ge(a, L, &L->c.done_seq, i - 3, ErrDrain, i)) return;
    // the interleaved attention tile waits for its pages one by one (t.ilv)
    for (int pg = 0; pg < (t.ilv ? 0 : t.npages); ++pg) {
      const int sq = first + pg;
      if (!wait_lds_ge(a, L, &L->c.slot_full[sq % LT::NP], sq / LT::NP + 1, ErrPage, i)) return;
    }
    if (tr && lane == 0) tr[8 + cw] = now_ticks();
    // hand the tile's pages back to the loaders once every LDS read of them has
    // returned (the loaders wait for kNW per use of a slot): one non-returning
    // add per lane, lane p < npages releasing page p, the others adding zero to
    // a word of their own (no divergent branch, so values held in registers
    // across the loop need no copies here)
    auto release = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const bool mine = lane < t.npages;
      LDS int* p = mine ? &L->c.slot_rel[(first + lane) % LT::NP] : &L->c.rel_sink[lane];
      __hip_atomic_fetch_add(p, mine ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    LdsSrc src;
    src.ring = lds_addr(&L->ring[0][0]);
    src.first = (uint32_t)(first % LT::NP) * kPage;
    src.off1 = (uint32_t)t.off1;
    src.wrap = (uint32_t)(LT::NP * kPage);
    const int sl = i & 3;
    const bool gemv = LT::GLM ? glm_is_gemm(op) : is_gemv(op);
    if constexpr (LT::GLM) {
      // weights (if any) are in the ring; activations follow the event
      if (!wait_lds_ge(a, L, &L->c.ready_seq, i + 1, ErrReady, i)) return;
      if (cw == 0 && tr && lane == 0) tr[1] = now_ticks();
      // the row ops' sum of squares over the four compute waves: each posts its
      // partial in its slot of the instruction and counts itself in, then all add
      // the four in wave order
      auto xsum = [&](float v) {
        if (lane == 0) {
          L->c.ssp[sl][cw][0] = v;
          __hip_atomic_fetch_add(&L->c.xch[sl], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (!wait_lds_ge(a, L, &L->c.xch[sl], kNW, ErrReady, i)) return v;  // aborting
        return ((L->c.ssp[sl][0][0] + L->c.ssp[sl][1][0]) + L->c.ssp[sl][2][0]) + L->c.ssp[sl][3][0];
      };
      if (gemv) {
        glm_gemm_wave(src, m, a.c, cw, &L->c.part[sl][cw][0], cw == 0 ? tr : nullptr);
      } else if (op == OpGA0) {
        glm_a0_wave(m, a.c, cw, xsum, cw == 0 ? tr : nullptr);
      } else if (op == OpGQaNorm) {
        glm_qan_wave(m, a.c, cw, xsum);
      } else if (op == OpGGateRed) {
        glm_gate_red_wave(m, a.c, cw);
      }
      release();
    } else if (gemv && !LT::MB) {
      const GemvIn gi = gemv_input(m, a.c);
      bool live = true;
      auto pre = [&]() {
        if (!wait_lds_ge(a, L, &L->c.ready_seq, i + 1, ErrReady, i)) {
          live = false;
          return false;
        }
        if (cw == 0 && tr && lane == 0) tr[1] = now_ticks();
        const bool load = m.w(WOpRow) != act_row;
        act_row = m.w(WOpRow);
        return load;
      };
      gemv_rows(src, act, gi, cw, &L->c.part[sl][cw][0], release, pre);
      if (!live) return;
      if (lane == 0) L->c.ssp[sl][cw][0] = act.ssw;
      if (cw == 0 && tr && lane == 0) tr[7] = now_ticks();
    } else {
      if (!wait_lds_ge(a, L, &L->c.ready_seq, i + 1, ErrReady, i)) return;
      if (cw == 0 && tr && lane == 0) tr[1] = now_ticks();
      if (gemv) {
        const GemvIn gi = gemv_input(m, a.c);
        LDS float* pw = &L->c.part[sl][cw][0];
        LDS float* sw = &L->c.ssp[sl][cw][0];
        if (LT::SETS > 1 && gemv_k_halves(op, a.c)) {
          if (own) {
            // first half; the helping group hands the pages back
            gemv_rows_mb(src, gi, a.c.B, a.c.V, cw, pw, sw, [] {}, 0, 2);
          } else {
            // second half: once the owning group has arrived (its partial
            // sums are in the slot and it has finished reading the pages),
            // release the pages and add to its sums
            bool live = true;
            auto rel2 = [&]() {
              if (!wait_lds_ge(a, L, &L->c.arrive[sl], kNW, ErrDrain, i)) {
                live = false;
                return;
              }
              release();
            };
            gemv_rows_mb(src, gi, a.c.B, a.c.V, cw, pw, sw, rel2, 1, 2);
            if (!live) return;
          }
        } else {
          gemv_rows_mb(src, gi, a.c.B, a.c.V, cw, pw, sw, release);
        }
      } else if (op == OpAttn) {
        if constexpr (LT::MB && HD == 64) {
          static_assert((LT::NP & (LT::NP - 1)) == 0, "the interleaved attention tile needs a power-of-two ring");
          // the group's rendezvous: all four compute waves past point k
          bool live = true;
          auto sync = [&](int k) {
            if (lane == 0) __hip_atomic_fetch_add(&L->c.xch[sl], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (!wait_lds_ge(a, L, &L->c.xch[sl], k * kNW, ErrReady, i)) live = false;
          };
          // the task's pages, waited for and handed back round by round
          struct Pages {
            const KArgs& a;
            LDS LT* L;
            int first, i, lane;
            bool& live;
            __device__ bool wait(int p) const {
              const int sq = first + p;
              if (!wait_lds_ge(a, L, &L->c.slot_full[sq % LT::NP], sq / LT::NP + 1, ErrPage, i)) live = false;
              return live;
            }
            __device__ void release(int p0, int p1) const {
              asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
              const bool mine = p0 + lane < p1;
              LDS int* p = mine ? &L->c.slot_rel[(first + p0 + lane) % LT::NP] : &L->c.rel_sink[lane];
              __hip_atomic_fetch_add(p, mine ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          } pages{a, L, first, i, lane, live};
          LdsAttnSrc asrc;
          asrc.ring = src.ring;
          asrc.first = src.first;
          asrc.mask = (uint32_t)(LT::NP * kPage - 1);
          attn_mfma64(asrc, m, a.c, cw, &L->c.scratch[set * kNW][0], &L->c.part[sl][0][0], cw == 0, sync, pages,
                      cw == 0 ? tr : nullptr);
          if (!live) return;
        } else {
          attn_wave<HD>(src, m, a.c, cw, L->c.scratch[set * kNW + cw], cw == 0, cw == 0 ? tr : nullptr);
        }
      } else if (op == OpCombine) {
        combine_wave<HD>(m, a.c, cw, cw == 0 ? tr : nullptr);
      } else if (op == OpArgmax) {
        argmax_part(m, a.c, cw, &L->c.part[sl][cw][0]);
      }
      if (!gemv && !t.ilv) release();
    }
    if (tr && lane == 0) tr[12 + cw] = now_ticks();
    // arrival: GEMV partials are in LDS; other ops stored their results to
    // global memory themselves, and the storer's counter add must not overtake
    // those stores.  A workgroup-scope release does not wait for them on this
    // target (the workgroup shares one CU, so it orders only LDS), and the
    // storer's own vmcnt wait covers only its own stores: each compute wave
    // waits for its stores to complete before it arrives.
    if (!gemv) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(&L->c.arrive[sl], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
}

template <int HD, bool MB, bool GLM = false>
__global__ void __launch_bounds__((LdsT<MB, GLM>::THREADS), 1) mk_megakernel(KArgs a) {
  typedef LdsT<MB, GLM> LT;
  __shared__ LT Ls;
  LDS LT* L = (LDS LT*)&Ls;
  {
    LDS int* c = (LDS int*)&L->c;
    const int n = (int)(sizeof(L->c) / 4);
    for (int k = threadIdx.x; k < n; k += blockDim.x) c[k] = 0;
  }
  // drop every line this CU's L1 and its XCD's L2 hold from before this launch,
  // so that the cached reads of this step's data (see CohT) cannot see a stale
  // copy; within the step no such line can appear
  if (threadIdx.x < 64) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
  // issue priority: the compute waves first, then the storer (the dependency
  // chain), the controller, and the loaders last
  const int w = threadIdx.x >> 6;
  if (w == 0) {
    __builtin_amdgcn_s_setprio(1);
    controller(a, L);
  } else if (w == 1) {
    __builtin_amdgcn_s_setprio(2);
    storer(a, L);
  } else if (w < 4) {
    loader(a, L, w - 2);
  } else {
    __builtin_amdgcn_s_setprio(3);
    compute<HD, LT>(a, L, (w - 4) % kNW, LT::SETS > 1 ? (w - 4) / kNW : 0);
  }
}

// ---------------------------------------------------------------------------
// Layerwise: one launch per operator, one workgroup (4 waves) per tile.
template <int HD, bool MB, bool GLM = false>
__global__ void __launch_bounds__(256) mk_layer_kernel(KArgs a, int num_cus, int first_task) {
  constexpr int PW = MB ? kMB * kMB : kMaxRows, SW = MB ? kMB : 1;
  __shared__ float part_s[kNW][PW];
  __shared__ float ssp_s[kNW][SW];
  __shared__ float scr_s[kNW][kScratch];
  LDS float(*part)[PW] = (LDS float(*)[PW])part_s;
  LDS float(*ssp)[SW] = (LDS float(*)[SW])ssp_s;
  LDS float(*scr)[kScratch] = (LDS float(*)[kScratch])scr_s;
  __shared__ uint32_t meta_s[64];
  const int t = first_task + blockIdx.x;
  const CST uint32_t* gins = (const CST uint32_t*)(uintptr_t)a.queue + ((size_t)(t % num_cus) * a.max_len + t / num_cus) * 32;
  const CST uint32_t* grow = (const CST uint32_t*)((const CST uint64_t*)(uintptr_t)a.optab + (size_t)gins[WOpRow] * 16);
  if (threadIdx.x < 32)
    meta_s[threadIdx.x] = gins[threadIdx.x];
  else if (threadIdx.x < 64)
    meta_s[threadIdx.x] = grow[threadIdx.x - 32];
  __syncthreads();
  const Meta m = load_meta((const LDS uint32_t*)meta_s);
  const int cw = threadIdx.x >> 6, lane = lane_id();
  const Tile tl = tile_info(m, a.c);
  GlbSrc src;
  src.p0 = tl.p0;
  src.p1 = tl.p1 ? tl.p1 : tl.p0;
  const int op = m.w(WOpcode);
  if constexpr (GLM) {
    if (glm_is_gemm(op)) {
      glm_gemm_wave<0>(src, m, a.c, cw, part[cw]);
      __syncthreads();
      if (cw == 0) glm_epilogue(m, a.c, &part[0][0]);
    } else {
      // sum of squares over the four waves of the block, added in wave order
      auto xsum = [&](float v) {
        if (lane == 0) ssp[cw][0] = v;
        __syncthreads();
        return ((ssp[0][0] + ssp[1][0]) + ssp[2][0]) + ssp[3][0];
      };
      if (op == OpGA0)
        glm_a0_wave(m, a.c, cw, xsum);
      else if (op == OpGQaNorm)
        glm_qan_wave<0>(m, a.c, cw, xsum);
      else if (op == OpGGateRed)
        glm_gate_red_wave<0>(m, a.c, cw);
    }
    return;
  }
  if (cw == 0) check_tokens(a, m);
  if (is_gemv(op)) {
    const GemvIn gi = gemv_input(m, a.c);
    if constexpr (MB) {
      if (gemv_k_halves(op, a.c)) {
        gemv_rows_mb<0>(src, gi, a.c.B, a.c.V, cw, part[cw], ssp[cw], [] {}, 0, 2);
        gemv_rows_mb<0>(src, gi, a.c.B, a.c.V, cw, part[cw], ssp[cw], [] {}, 1, 2);
      } else {
        gemv_rows_mb<0>(src, gi, a.c.B, a.c.V, cw, part[cw], ssp[cw], [] {});
      }
      __syncthreads();
      if (cw == 0) {
        ResMB res = gemv_residual_mb<0>(m, a.c);
        res.ss = gemv_sumsq_mb<0>(m, a.c);
        gemv_epilogue_mb(m, a.c, &part[0][0], &ssp[0][0], res);
      }
    } else {
      Act act;
      gemv_rows<0>(src, act, gi, cw, part[cw], [] {}, [] { return true; });
      if (lane == 0) ssp[cw][0] = act.ssw;
      __syncthreads();
      if (cw == 0) gemv_epilogue(m, a.c, part, &ssp[0][0], gemv_residual<0>(m, a.c));
    }
  } else if (op == OpAttn) {
    // (the batched megakernel runs its attention on the matrix cores; here the
    // vector form, which suits tasks read in place from device memory)
    attn_wave<HD, 0>(src, m, a.c, cw, scr[cw], cw == 0);
  } else if (op == OpCombine) {
    combine_wave<HD, 0>(m, a.c, cw);
  } else if (op == OpArgmax) {
    argmax_part<0>(m, a.c, cw, part[cw]);
    __syncthreads();
    if (cw == 0) argmax_final(m, &part[0][0], PW);
  }
}

template <bool MB>
const void* megakernel_fn(int hd) {
  return hd == 64 ? (const void*)mk_megakernel<64, MB> : (const void*)mk_megakernel<128, MB>;
}

}  // namespace

// ---- launch wrappers used by the host API ----------------------------------------
// Batch 1 runs the fp32 GEMV path; batch 2..16 the matrix-core path.
namespace mk {

hipError_t launch_megakernel(const KArgs& a, int num_cus, hipStream_t s) {
  if (a.c.glm) {
    hipLaunchKernelGGL((mk_megakernel<64, true, true>), dim3(num_cus), dim3(LdsT<true, true>::THREADS), 0, s, a);
  } else if (a.c.B == 1) {
    constexpr int T = LdsT<false>::THREADS;
    if (a.c.hd == 64)
      hipLaunchKernelGGL((mk_megakernel<64, false>), dim3(num_cus), dim3(T), 0, s, a);
    else
      hipLaunchKernelGGL((mk_megakernel<128, false>), dim3(num_cus), dim3(T), 0, s, a);
  } else {
    constexpr int T = LdsT<true>::THREADS;
    if (a.c.hd == 64)
      hipLaunchKernelGGL((mk_megakernel<64, true>), dim3(num_cus), dim3(T), 0, s, a);
    else
      hipLaunchKernelGGL((mk_megakernel<128, true>), dim3(num_cus), dim3(T), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_layer(const KArgs& a, int num_cus, int first_task, int ntasks, hipStream_t s) {
  if (a.c.glm) {
    hipLaunchKernelGGL((mk_layer_kernel<64, true, true>), dim3(ntasks), dim3(256), 0, s, a, num_cus, first_task);
  } else if (a.c.B == 1) {
    if (a.c.hd == 64)
      hipLaunchKernelGGL((mk_layer_kernel<64, false>), dim3(ntasks), dim3(256), 0, s, a, num_cus, first_task);
    else
      hipLaunchKernelGGL((mk_layer_kernel<128, false>), dim3(ntasks), dim3(256), 0, s, a, num_cus, first_task);
  } else {
    if (a.c.hd == 64)
      hipLaunchKernelGGL((mk_layer_kernel<64, true>), dim3(ntasks), dim3(256), 0, s, a, num_cus, first_task);
    else
      hipLaunchKernelGGL((mk_layer_kernel<128, true>), dim3(ntasks), dim3(256), 0, s, a, num_cus, first_task);
  }
  return hipGetLastError();
}

hipError_t megakernel_occupancy(int hd, int batch, bool glm, int* blocks_per_cu) {
  const void* f = glm ? (const void*)mk_megakernel<64, true, true>
                      : (batch == 1 ? megakernel_fn<false>(hd) : megakernel_fn<true>(hd));
  const int threads = glm ? LdsT<true, true>::THREADS : (batch == 1 ? LdsT<false>::THREADS : LdsT<true>::THREADS);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f, threads, 0);
}

int ring_pages(int batch) { return batch == 1 ? LdsT<false>::NP : LdsT<true>::NP; }

// Set-up of a decode step at new lengths, one launch: rewrites the payload
// words of queued instructions in place (patch i = (word index, three values)
// stores the values at queue[index .. index + 2]), installs the step's RoPE
// table (nr floats), and hands the previous step's next tokens (nt int32) to
// the token buffer and, if given, to the caller's output row.
__global__ void mk_step_setup(int* queue, const int4* patches, int n, float* rope, const float* rope_src, int nr,
                              int* tok, const int* next, int* out, int nt) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const int4 p = patches[i];
    queue[p.x] = p.y;
    queue[p.x + 1] = p.z;
    queue[p.x + 2] = p.w;
  }
  if (i < nr) rope[i] = rope_src[i];
  if (i < nt) {
    const int t = next[i];
    tok[i] = t;
    if (out) out[i] = t;
  }
}

hipError_t launch_step_setup(int* queue, const void* patches, int n, float* rope, const float* rope_src, int nr,
                             int* tok, const int* next, int* out, int nt, hipStream_t s) {
  const int m = n > nr ? (n > nt ? n : nt) : (nr > nt ? nr : nt);
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(mk_step_setup, dim3((m + 255) / 256), dim3(256), 0, s, queue, (const int4*)patches, n, rope,
                     rope_src, nr, tok, next, out, nt);
  return hipGetLastError();
}

}  // namespace mk

namespace {
// ---- streaming-read probe ----------------------------------------------------
// The ceiling of a plain weight stream on this device, the second denominator of
// the roofline: pages of 16 KiB are dealt round-robin to (workgroup, wave), and
// each wave reads its pages either with LDS-DMA into an LDS ring (as the
// megakernel's loaders do) or with 16-byte loads into registers, keeping DEPTH
// pages in flight.  Nothing is computed on the data; an XOR of the register
// loads goes to sink so that they are not removed.
template <int DEPTH>
__global__ void __launch_bounds__(512, 1) mk_stream_lds(const char* __restrict__ src, long npages, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) char ring[8][kPage];
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const long stride = (long)gridDim.x * nw;
  int k = 0;
  for (long p = (long)blockIdx.x * nw + w; p < npages; p += stride, ++k) {
    const GLB char* g = (const GLB char*)src + p * kPage + lane * 16;
    LDS char* dst = (LDS char*)ring[(w * DEPTH + k % DEPTH) & 7];
#pragma unroll
    for (int j = 0; j < 16; ++j)
      __builtin_amdgcn_global_load_lds((const GLB void*)(g + j * 1024), (lds_void*)(dst + j * 1024), 16, 0, kDmaNT);
    if (DEPTH == 1) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (DEPTH == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    if (DEPTH == 3) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    if (DEPTH == 4) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0 && k == -1) sink[0] = 0;
}

template <int DEPTH>
__global__ void __launch_bounds__(512, 1) mk_stream_vgpr(const char* __restrict__ src, long npages, unsigned* sink) {
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6, lane = threadIdx.x & 63;
  const long stride = (long)gridDim.x * nw;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long p0 = (long)blockIdx.x * nw + w; p0 < npages; p0 += stride * DEPTH) {
    u32x4 v[DEPTH][16];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const long p = p0 + d * stride < npages ? p0 + d * stride : p0;
      const GLB u32x4* g = (const GLB u32x4*)((const GLB char*)src + p * kPage) + lane;
#pragma unroll
      for (int j = 0; j < 16; ++j) v[d][j] = __builtin_nontemporal_load(g + j * 64);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc ^= v[d][j];
  }
  sink[(size_t)blockIdx.x * nw + w] = (acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u ? 1u : 0u;
}

}  // namespace

namespace mk {
hipError_t launch_stream_probe(const void* src, long npages, int lds_dma, int workgroups, int waves, int depth,
                               unsigned* sink, hipStream_t s) {
  const dim3 g(workgroups), b(64 * waves);
  const char* p = (const char*)src;
  if (lds_dma) {
    switch (depth) {
      case 1: hipLaunchKernelGGL(mk_stream_lds<1>, g, b, 0, s, p, npages, sink); break;
      case 2: hipLaunchKernelGGL(mk_stream_lds<2>, g, b, 0, s, p, npages, sink); break;
      case 3: hipLaunchKernelGGL(mk_stream_lds<3>, g, b, 0, s, p, npages, sink); break;
      default: hipLaunchKernelGGL(mk_stream_lds<4>, g, b, 0, s, p, npages, sink); break;
    }
  } else {
    switch (depth) {
      case 1: hipLaunchKernelGGL(mk_stream_vgpr<1>, g, b, 0, s, p, npages, sink); break;
      default: hipLaunchKernelGGL(mk_stream_vgpr<2>, g, b, 0, s, p, npages, sink); break;
    }
  }
  return hipGetLastError();
}
}  // namespace mk
