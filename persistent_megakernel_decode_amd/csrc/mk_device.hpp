// Device-side definitions shared by the persistent interpreter and the
// layerwise kernels: constants, instruction decoding, tile byte layout and the
// tile arithmetic of every operator of the Llama-family decode step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// LDS (address space 3): device code reaches shared memory only through such
// pointers so that every access is a ds_* instruction, never a flat access
// that would queue in the vector-memory pipeline behind the page DMA.
#define LDS __attribute__((address_space(3)))
// Global memory (address space 1): pointers taken from the operand table are
// cast to it so loads and stores are global_* (vmcnt only), not flat_*.
#define GLB __attribute__((address_space(1)))
// Constant address space (4): the instruction queue and the operand table are
// never written while a kernel runs; reading them through such pointers gives
// scalar loads (the scalar cache), which do not queue in the vector-memory
// pipeline behind the weight stream.
#define CST __attribute__((address_space(4)))
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace mkd {

// ---- instruction words (same layout as the host planner) -------------------
enum : int {
  WOpcode = 0, WSpec = 1, WOpRow = 2, WWaitCnt = 3, WWaitEv = 4, WWaitTgt = 5, WSigCnt = 6, WSigEv = 7,
  WSigInc = 8, WTask = 9, WLayer = 10, WGx = 11, WGy = 12, WGz = 13, WPay = 14,
  // second wait (event, target) and second signal (event, increment): word 3 /
  // word 6 count the waits / signals, 0..2
  WWait2Ev = 24, WWait2Tgt = 25, WSig2Ev = 26, WSig2Inc = 27,
  // LDS copy only (the queue holds zero there): sequence number of the
  // instruction's first ring page, written by the controller as it stages it
  WFirstPage = 31
};
enum : int { OpNoop = 0, OpQkv = 1, OpAttn = 2, OpCombine = 3, OpOproj = 4, OpGateUp = 5, OpDown = 6, OpLmHead = 7, OpArgmax = 8 };
// GLM-style pre-attention path: add + RMSNorm + fp8 quant (one token row per
// task), fp8 GEMM tiles of 16 weight rows (QKV-A, head gate, indexer-K, QKV-B,
// indexer-Q) and the q path's RMSNorm + requant with the KV-row write.
enum : int { OpGA0 = 9, OpGQkva = 10, OpGGate = 11, OpGIdxk = 12, OpGQaNorm = 13, OpGQkvb = 14, OpGIdxq = 15,
             OpGGateRed = 16 };

// ---- operand table slots (one row of 16 u64 per op) --------------------------
enum : int {
  // Batch > 1: the GEMV activations are stored pre-split (see act_split):
  // the producer of a normed input also stores it times the consumer's
  // RMSNorm weight (QkvPrep, GuPrep, LmPrep) and per-chunk sums of squares
  // (QkvSs, GuSs, LmSs); the attention output and the FFN activation are
  // stored only in that form (OIn, DnIn).
  // QKV
  QkvWq = 0, QkvWk = 1, QkvWv = 2, QkvNorm = 3, QkvX = 4, QkvEmbed = 5, QkvTokens = 6, QkvOut = 7, QkvPrep = 8,
  QkvSs = 9,
  // ATTN
  AttnQkv = 0, AttnK = 1, AttnV = 2, AttnRope = 3, AttnOut = 4, AttnQn = 5, AttnKn = 6,
  // COMBINE
  CombPart = 0, CombOut = 1,
  // OPROJ (OPrepW / OPrep / OSs: the gate/up input's norm weight, pre-split
  // copy and chunk sums of squares, batch > 1)
  OWo = 0, OIn = 1, OX = 2, OEmbed = 3, OTokens = 4, OOut = 5, OPrepW = 6, OPrep = 7, OSs = 8,
  // GATEUP
  GuWg = 0, GuWu = 1, GuNorm = 2, GuIn = 3, GuOut = 4, GuPrep = 5, GuSs = 6,
  // DOWN (DnPrepW / DnPrep / DnSs: the same for the next QKV or the LM head)
  DnW = 0, DnIn = 1, DnRes = 2, DnOut = 3, DnPrepW = 4, DnPrep = 5, DnSs = 6,
  // LMHEAD
  LmW = 0, LmNorm = 1, LmIn = 2, LmLogits = 3, LmMax = 4, LmPrep = 5, LmSs = 6,
  // ARGMAX
  AmMax = 0, AmOut = 1,
  // GLM A0: inputs x, r (bf16), norm weight, outputs r_out (bf16), norm (fp32), codes, scales
  GaX = 0, GaR = 1, GaNorm = 2, GaROut = 3, GaN = 4, GaA8 = 5, GaAS = 6,
  // GLM fp8 GEMMs: weight codes and block scales, activation codes and scales
  // (or the fp32 norm output for the gate), output, RoPE table, token rows info
  GmW = 0, GmS = 1, GmA8 = 2, GmAS = 3, GmAF = 4, GmOut = 5, GmRope = 6, GmRows = 7,
  // GLM q-path norm: QKV-A output, q / kv norm weights, q codes and scales, KV cache, RoPE, rows
  QnIn = 0, QnNorm = 1, QnKvNorm = 2, QnA8 = 3, QnAS = 4, QnKv = 5, QnRope = 6, QnRows = 7,
  // GLM head-gate reduce: the K-split partials, the gate output
  GrPart = 0, GrOut = 1
};

constexpr int kPage = 16384;  // bytes per LDS page
constexpr int kNumPages = 9;  // page ring of the interpreter: 144 KiB
constexpr int kNW = 4;        // compute waves per workgroup (K split / one q head each)
constexpr int kMaxRows = 16;  // weight rows per GEMV tile
constexpr int kMB = 16;       // sequences per batched GEMV tile (the MFMA N dimension)
constexpr int kMaxChunks = 6; // 16-byte activation chunks per lane (K / (8 * kNW * 64))
constexpr int kScratch = 384; // floats of per-compute-wave scratch (attention: 3 head vectors)
constexpr int kTraceWords = 16; // timestamps per traced instruction
constexpr int kCtrStride = 64;  // u32 words between event counters: one 256-byte line each
// Each event is counted in kCtrSub sub-counters (a producer on compute unit c
// adds to sub-counter c mod kCtrSub; a waiter sums all of them), so the atomic
// adds of one event's many producers do not serialize on one line: the adds of
// one line are applied one after another at the memory side, and the waiters'
// polls queue behind them (Llama-1B batch 1: 16 lines 883 us, 32 845, 64 828).
// Sub-counter k of event e is word ctr_word(e, k, E) of the counter buffer: an
// event's lines are contiguous (one 16 KiB block), so a poll touches one small
// range (Llama-1B 830 -> 807 us against the lines of one k being contiguous).
constexpr int kCtrSub = 64;
constexpr int kCtrPer = kCtrSub > 64 ? kCtrSub / 64 : 1;  // sub-counters a polling lane reads
static_assert(kCtrSub <= 64 || kCtrSub % 64 == 0, "sub-counters: up to 64, or a multiple of 64");
__host__ __device__ inline size_t ctr_word(int e, int k, int num_events) {
  (void)num_events;
  return ((size_t)e * kCtrSub + k) * kCtrStride;
}

struct Consts {
  int H, nq, nkv, hd, F, V, L, B, cap, hpg, RPG, S, T_v, qk_norm;
  float eps, inv_sqrt_hd;
  // GLM path (glm != 0): q_lora, kv_lora, rope dims, nope dims per head, QKV-A
  // outputs, gate outputs, indexer head dim, indexer-Q outputs
  int glm, ql, kl, rd, nope, na, ng, nik, niq;
  // batch > 1: rows per stored sum of squares of the residual stream (8, 4, 2
  // or 1; stored [K / 8][B][8 / rows]) for the QKV / LM-head input (written by
  // down) and for gate/up's (written by O)
  int ssg_a, ssg_f;
};

struct KArgs {
  const int* queue;           // [C][max_len][32]
  const uint64_t* optab;      // [num_ops][16]
  unsigned* counters;         // [num_events][kCtrSub] lines (ctr_word)
  int num_events;
  unsigned* err;              // watchdog record [8]
  unsigned long long* trace;  // [C][max_len][kTraceWords] or null
  int max_len;
  int dma_pages;  // pages in flight per loader wave (1 to 3; batch-1 interpreter)
  unsigned epoch;
  unsigned run_id;  // sequence number of the run (megakernel or layerwise), for err[7]
  unsigned long long timeout_ticks;
  Consts c;
};

// ---- small helpers -----------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Element (b, k) of a [B][K] activation of this step (the residual stream,
// the attention output, the FFN activation): laid out as [K / 8][B][8], so
// that the 16 sequences' 32-byte chunks of one k range are contiguous and a
// batched tile's loads of a k-step cover one 2 KiB run instead of B lines a
// power-of-two row length apart.  At B = 1 this is the plain vector.
__device__ __forceinline__ size_t act_ix(int b, int k, int B) {
  return ((size_t)(k >> 3) * B + b) * 8 + (k & 7);
}
// The pre-split form of such an activation (batch > 1): per 8-element chunk
// and sequence 32 bytes, the chunk's bf16 high parts h = bf16(v) then its low
// parts bf16(v - h) -- the two matrix-core operands of a batched tile, so that
// the tiles that read it convert nothing.  Byte offset of element (b, k)'s
// high part; its low part sits 16 bytes further.
__device__ __forceinline__ uint32_t split_off(int b, int k, int B) {
  return (uint32_t)((((k >> 3) * B + b) * 32) + (k & 7) * 2);
}
// Store v in that form (16-bit stores written through to the device's
// coherence point, like st_agent).
__device__ __forceinline__ void st_split(const GLB void* base, int b, int k, int B, float v) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, 0x7FFFFFFF, 0x00020000);
  const __bf16 h = (__bf16)v;
  const __bf16 l = (__bf16)(v - (float)h);
  const uint32_t o = split_off(b, k, B);
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, h), r, (int)o, 0, 16 /* sc1 */);
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, l), r, (int)o + 16, 0, 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Cross-lane reductions with DPP (register-to-register lane moves, no LDS):
// quad_perm [1,0,3,2] and [2,3,0,1] (xor 1, xor 2), row_half_mirror (i -> 7-i
// within 8 lanes), row_ror 4 / 8 (rotate within 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
enum : int { DppXor1 = 0xB1, DppXor2 = 0x4E, DppHalfMirror = 0x141, DppRor4 = 0x124, DppRor8 = 0x128 };
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// every lane of each 16-lane row ends with the row's sum
__device__ __forceinline__ float row_sum16(float v) {
  v += dppf<DppXor1>(v);
  v += dppf<DppXor2>(v);
  v += dppf<DppRor4>(v);
  v += dppf<DppRor8>(v);
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dppf<DppXor1>(v));
  v = fmaxf(v, dppf<DppXor2>(v));
  v = fmaxf(v, dppf<DppRor4>(v));
  v = fmaxf(v, dppf<DppRor8>(v));
  return v;
}
// sum over the lanes that hold sub-counters (integer, wave-uniform): row sums
// by DPP, then the rows' totals
__device__ __forceinline__ unsigned ctr_sum_u32(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, DppXor1, 0xF, 0xF, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, DppXor2, 0xF, 0xF, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, DppRor4, 0xF, 0xF, false);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, DppRor8, 0xF, 0xF, false);
  unsigned r = (unsigned)__builtin_amdgcn_readlane((int)v, 0);
  if (kCtrSub > 16) r += (unsigned)__builtin_amdgcn_readlane((int)v, 16);
  if (kCtrSub > 32) r += (unsigned)__builtin_amdgcn_readlane((int)v, 32) + (unsigned)__builtin_amdgcn_readlane((int)v, 48);
  return r;
}
// wave-uniform sum / max of one value per lane
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row_max16(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Data one compute unit writes for another within a step is stored agent-coherent
// (a relaxed agent-scope atomic store: written through the XCD's L2), so a
// producer never needs the L2 write-back that an agent-scope release fence
// performs -- under full HBM load that write-back costs tens of microseconds.
// The producer then only waits for its stores to complete before its counter
// atomic; consumers still acquire.
__device__ __forceinline__ void st_agent(GLB float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(GLB int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes per lane at base + off (base wave-uniform, off per lane, 16-byte
// aligned), with the cache policy of st_agent (sc1: written through to the
// device's coherence point): one store instruction instead of four scattered
// ones, for lanes that own four consecutive fp32 outputs.
__device__ __forceinline__ void st_agent16(const GLB void* base, uint32_t off, f32x4 v) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, 0x7FFFFFFF, 0x00020000);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 16 /* sc1 */);
}
// Reads of data that other compute units wrote during the same step
// (activations, residual stream, q/k/v, attention partials, LM tile maxima,
// quantized activations and scales).  The producers store them agent-coherent
// and count them only once the stores have completed, and the interpreter waits
// for an event without an acquire that would invalidate the L2 (one per
// instruction costs about 80 us per step and throws away every other CU's
// cached lines on that XCD).  A consumer may then read through the caches
// (POL = 0) only data that cannot sit stale in them: the interpreter
// invalidates its L1 / L2 once when it starts, and such a buffer is written
// once per step, read only after the event that counts all of its producers,
// and shares no cache line with data of another event (per-layer slices start
// on 256-byte boundaries).  Data that fails the last condition -- the attention
// partials, whose (sequence, kv head) blocks are not line-aligned and complete
// under different events -- is read with sc1 loads (POL = kCohPolicy), served
// at the device's coherence point.  The descriptor's base must be wave-uniform
// (per-lane parts go into the offset); its 2 GiB range is never reached.
constexpr int kCohPolicy = 16;  // sc1
template <int POL>
struct CohT {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ explicit CohT(const GLB void* base) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    r = __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0, 0x7FFFFFFF,
                                          0x00020000);
  }
  __device__ __forceinline__ f32x4 f4(uint32_t off) const {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL));
  }
  __device__ __forceinline__ u32x4 u4(uint32_t off) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POL));
  }
  __device__ __forceinline__ f32x2 f2(uint32_t off) const {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POL));
  }
  __device__ __forceinline__ float f1(uint32_t off) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, POL));
  }
  // per-lane offset plus a wave-uniform one (kept in a scalar register)
  __device__ __forceinline__ float f1(uint32_t voff, uint32_t soff) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, POL));
  }
};

// token id of sequence 0, clamped into [0, vocab) so that a bad id cannot index
// outside the embedding (the run is flagged as failed: see check_tokens)
__device__ __forceinline__ int token_of(const GLB int* tokens, int b, int V) {
  const int t = tokens[b];
  return t < 0 ? 0 : (t >= V ? V - 1 : t);
}
__device__ __forceinline__ int token0(const uint64_t tokens_ptr, int V) {
  int t = ((const GLB int*)tokens_ptr)[0];
  return t < 0 ? 0 : (t >= V ? V - 1 : t);
}
__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ---- instruction metadata ---------------------------------------------------------
// An instruction's 32 words and its operand-table row (16 u64) form a 64-dword
// record.  The interpreter's waves read it from a copy in LDS with one load per
// lane (lane l holds dword l) and take fields out with v_readlane, which
// returns them wave-uniform (in scalar registers) without further memory
// round trips.  The loader reads the records straight from device memory.
struct Meta {
  uint32_t v;  // lane l < 32: instruction word l; lane 32 + j: dword j of the operand row
  __device__ __forceinline__ int w(int k) const { return __builtin_amdgcn_readlane((int)v, k); }
  __device__ __forceinline__ uint64_t q(int k) const {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)v, 33 + 2 * k) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)v, 32 + 2 * k);
  }
};
__device__ __forceinline__ Meta load_meta(const LDS uint32_t* rec) {
  Meta m;
  m.v = rec[threadIdx.x & 63];
  return m;
}
// The same fields through scalar loads from the queue and the operand table.
struct GMeta {
  const CST int* ins;
  const CST uint64_t* row;
  __device__ __forceinline__ int w(int k) const { return ins[k]; }
  __device__ __forceinline__ uint64_t q(int k) const { return row[k]; }
};

// ---- tile byte layout ---------------------------------------------------------
// A tile's weight bytes are one or two contiguous source segments placed one
// after the other in the tile's buffer, the second at a 1 KiB boundary.  Plain
// scalars (no arrays) so that nothing is indexed at run time and everything
// stays in registers.
struct Tile {
  const GLB char* p0;
  const GLB char* p1;
  int len0, off1, len1;
  int bytes, npages;
  // segment 0 as rows of seglen bytes, stride bytes apart in memory (packed
  // densely in the tile); stride 0: one contiguous run
  int seglen, stride;
  // batched head_dim-64 attention: the K and V rows interleaved in chunks of
  // 32 positions (4 KiB of K rows, then the same positions' 4 KiB of V rows),
  // so that the task can consume and hand back its pages in position order
  // and may be longer than the ring (attn_mfma64)
  int ilv;
};

__device__ __forceinline__ int round1k(int v) { return (v + 1023) & ~1023; }

template <class M>
__device__ inline Tile tile_info(const M& m, const Consts& c) {
  Tile t;
  t.p0 = nullptr;
  t.p1 = nullptr;
  t.len0 = t.off1 = t.len1 = 0;
  t.seglen = t.stride = 0;
  t.ilv = 0;
  const int op = m.w(WOpcode);
  switch (op) {
    case OpQkv: {
      const int g = m.w(WGx), row0 = m.w(WPay), nrows = m.w(WPay + 1);
      const int qrows = c.hpg * c.hd;
      if (row0 < qrows)
        t.p0 = (const GLB char*)m.q(QkvWq) + ((size_t)g * qrows + row0) * c.H * 2;
      else if (row0 < qrows + c.hd)
        t.p0 = (const GLB char*)m.q(QkvWk) + ((size_t)g * c.hd + row0 - qrows) * c.H * 2;
      else
        t.p0 = (const GLB char*)m.q(QkvWv) + ((size_t)g * c.hd + row0 - qrows - c.hd) * c.H * 2;
      t.len0 = nrows * c.H * 2;
      break;
    }
    case OpOproj:
      t.p0 = (const GLB char*)m.q(OWo) + (size_t)m.w(WPay) * c.nq * c.hd * 2;
      t.len0 = m.w(WPay + 1) * c.nq * c.hd * 2;
      break;
    case OpGateUp:
      t.p0 = (const GLB char*)m.q(GuWg) + (size_t)m.w(WPay) * c.H * 2;
      t.p1 = (const GLB char*)m.q(GuWu) + (size_t)m.w(WPay) * c.H * 2;
      t.len0 = t.len1 = m.w(WPay + 1) * c.H * 2;
      break;
    case OpDown:
      t.p0 = (const GLB char*)m.q(DnW) + (size_t)m.w(WPay) * c.F * 2;
      t.len0 = m.w(WPay + 1) * c.F * 2;
      break;
    case OpLmHead:
      t.p0 = (const GLB char*)m.q(LmW) + (size_t)m.w(WPay) * c.H * 2;
      t.len0 = m.w(WPay + 1) * c.H * 2;
      break;
    case OpGGate: {
      // a K-split of 16 rows: blocks [kb0, kb0 + nkb) of 128 columns, each row's
      // part contiguous (nkb * 128 bytes), the rows c.H bytes apart
      const int row0 = m.w(WPay), nrows = m.w(WPay + 1), kb0 = m.w(WPay + 3), nkb = m.w(WPay + 4);
      t.p0 = (const GLB char*)m.q(GmW) + (size_t)row0 * c.H + kb0 * 128;
      t.seglen = nkb * 128;
      t.stride = c.H;
      t.len0 = nrows * t.seglen;
      break;
    }
    case OpGQkva:
    case OpGIdxk:
    case OpGQkvb:
    case OpGIdxq: {
      // fp8 weight rows [row0, row0 + nrows) and, for a RoPE-pair tile, the
      // same number of rows from row1 as the second segment
      const int K = (op == OpGQkvb || op == OpGIdxq) ? c.ql : c.H;
      const int row0 = m.w(WPay), nrows = m.w(WPay + 1), row1 = m.w(WPay + 2);
      t.p0 = (const GLB char*)m.q(GmW) + (size_t)row0 * K;
      t.len0 = nrows * K;
      if (row1 >= 0) {
        t.p1 = (const GLB char*)m.q(GmW) + (size_t)row1 * K;
        t.len1 = nrows * K;
      }
      break;
    }
    case OpAttn: {
      const int b = m.w(WGx), g = m.w(WGy), lo = m.w(WPay), hi = m.w(WPay + 1), pos = m.w(WPay + 2);
      int nk = (hi < pos ? hi : pos) - lo;
      if (nk < 0) nk = 0;
      const size_t base = (((size_t)b * c.nkv + g) * c.cap + lo) * c.hd * 2;
      t.p0 = (const GLB char*)m.q(AttnK) + base;
      t.p1 = (const GLB char*)m.q(AttnV) + base;
      t.len0 = t.len1 = nk * c.hd * 2;
      t.ilv = c.B > 1 && c.hd == 64;
      break;
    }
    default:
      break;
  }
  t.off1 = round1k(t.len0);
  t.bytes = t.ilv ? ((t.len0 + 4095) >> 12) * 8192 : t.len1 ? t.off1 + t.len1 : t.len0;
  t.npages = (t.bytes + kPage - 1) / kPage;
  return t;
}

// ---- weight sources -------------------------------------------------------------
// LDS page ring: page j of the tile lives in ring slot (first + j) mod kNumPages,
// so tile byte t sits at ring offset (first * kPage + t) mod (kNumPages * kPage).
// The tile spans at most kNumPages pages, so the modulo is one conditional
// subtraction: min over unsigned of x and x - ring size (the second wraps to a
// huge value while x is below the ring size).  The uniform part of x is scalar.
struct LdsSrc {
  static constexpr bool kLds = true;  // tiles packed densely (strided rows become rows of their own length)
  uint32_t ring;   // LDS byte address of ring slot 0
  uint32_t first;  // first * kPage
  uint32_t off1;   // tile offset of segment 1
  uint32_t wrap;   // ring size in bytes
  __device__ __forceinline__ uint32_t addr(int seg, uint32_t o) const {
    const uint32_t x = first + (seg ? off1 : 0u) + o;
    const uint32_t y = x - wrap;
    return ring + (x < y ? x : y);
  }
  __device__ __forceinline__ uint4 ld16(int seg, int o) const {
    const u32x4 v = *(const LDS u32x4*)(uintptr_t)addr(seg, (uint32_t)o);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ uint16_t ld2(int seg, int o) const {
    return *(const LDS uint16_t*)(uintptr_t)addr(seg, (uint32_t)o);
  }
  __device__ __forceinline__ uint32_t ld4(int seg, int o) const {
    return *(const LDS uint32_t*)(uintptr_t)addr(seg, (uint32_t)o);
  }
};
// The interleaved attention tile (Tile::ilv) in a power-of-two ring: row byte o
// of segment s (0 K, 1 V) sits at tile offset o + ((o >> 12) + s) * 4096, and
// the tile may be longer than the ring (its pages are handed back as the task
// moves on), so the ring offset is taken modulo the ring size.
struct LdsAttnSrc {
  uint32_t ring;   // LDS byte address of ring slot 0
  uint32_t first;  // first * kPage
  uint32_t mask;   // ring size in bytes - 1
  __device__ __forceinline__ uint32_t addr(int seg, uint32_t o) const {
    return ring + ((first + o + (((o >> 12) + (uint32_t)seg) << 12)) & mask);
  }
  __device__ __forceinline__ uint4 ld16(int seg, int o) const {
    const u32x4 v = *(const LDS u32x4*)(uintptr_t)addr(seg, (uint32_t)o);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};
// A tile whose pages do not wrap around the ring end: plain offsets.
struct LdsLin {
  uint32_t base;  // LDS byte address of the tile's first page
  uint32_t off1;
  __device__ __forceinline__ uint4 ld16(int seg, int o) const {
    const u32x4 v = *(const LDS u32x4*)(uintptr_t)(base + (seg ? off1 : 0u) + (uint32_t)o);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
};
// Straight from device memory (layerwise kernels).
struct GlbSrc {
  static constexpr bool kLds = false;  // tiles read in place (row stride of the weight matrix)
  const GLB char* p0;
  const GLB char* p1;
  __device__ __forceinline__ uint4 ld16(int seg, int o) const {
    const u32x4 v = *(const GLB u32x4*)((seg ? p1 : p0) + o);
    return make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ uint16_t ld2(int seg, int o) const { return *(const GLB uint16_t*)((seg ? p1 : p0) + o); }
  __device__ __forceinline__ uint32_t ld4(int seg, int o) const { return *(const GLB uint32_t*)((seg ? p1 : p0) + o); }
};

// Which activation and norm a GEMV op reads, and its K.
struct GemvIn {
  const GLB float* xf;
  const GLB uint16_t* xb;
  const GLB uint16_t* nw;
  const GLB uint16_t* emb;  // embedding table when the input is the token's row (xf null)
  const GLB int* tok;       // token ids [B]
  const GLB char* xs;    // batch > 1: the input in pre-split form (act_split)
  const GLB float* ssc;  // with xs and a fused norm: sums of squares [K / 8][B][8 / ssg]
  int ssg;               // rows per sum
  int K;
  int n0, nrows;  // rows in segment 0, total rows
  int norm;       // the op fuses an RMSNorm (scale applied in the epilogue)
};

// ---- activations of a GEMV tile ---------------------------------------------
// Each compute wave owns about K / kNW consecutive input elements; lane l holds the
// 16-byte chunks l, l + 64, ... of that range (times the RMSNorm weight when the
// op fuses a norm) as bf16 pairs, x[j][0..3] the high parts h = bf16(x) and
// x[j][4..7] the low parts bf16(x - h), for v_dot2 against the bf16 weights:
// exact products, fp32 accumulation, h + l keeps about 16 bits of x, and half
// the VALU instructions of unpacking the weights for fp32 FMAs (Qwen3-8B 3851 ->
// 3758 us; Llama-1B, whose tiles are not bound by the GEMV, 793 -> 798).  Plus
// the lane's partial sum of squares of the fp32 inputs.
struct Act {
  float x[kMaxChunks][8];  // bf16 pairs, bit-cast
  float ss;   // this lane's sum of squares of the (un-normed) inputs
  float ssw;  // the wave's sum of ss
  int nc;
};
__device__ __forceinline__ bf16x2 act_pair(const Act& a, int j, int k) { return __builtin_bit_cast(bf16x2, a.x[j][k]); }

// src: fp32 vector (xf) or a bf16 row (xb); nw: bf16 norm weight or null.
// All loads are issued before any is used (addresses of chunks outside the
// wave's range are clamped to chunk 0 and their values zeroed afterwards); the
// fp32 input lands straight in a.x, so besides a the load holds only the norm
// weights (and a bf16 input) in flight: it can run while a GEMV tile's weights
// sit in registers.  MC: chunks per lane unrolled (at least a.nc).
template <int MC, int POL = 0>
__device__ inline void load_act_t(Act& a, int K, int cw, const GLB float* xf, const GLB uint16_t* xb,
                                  const GLB uint16_t* nw) {
  const int lane = lane_id();
  const int nch = K / 8;                    // 16-byte chunks of bf16 weights per row
  const int cpw = (nch + kNW - 1) / kNW;    // chunks per wave (the last wave may get fewer)
  const int base = cw * cpw;
  a.nc = (cpw + 63) / 64;
  u32x4 xr[MC], wr[MC];
  float xf4[MC][8];
  bool ok[MC];
#pragma unroll
  for (int j = 0; j < MC; ++j) {
    const int ch = lane + 64 * j;
    ok[j] = j < a.nc && ch < cpw && base + ch < nch;
    const int k0 = (ok[j] ? base + ch : 0) * 8;
    if (j < a.nc) {
      if (xf) {
        const CohT<POL> cx(xf);
        const f32x4 v0 = cx.f4(k0 * 4), v1 = cx.f4(k0 * 4 + 16);
        xf4[j][0] = v0.x; xf4[j][1] = v0.y; xf4[j][2] = v0.z; xf4[j][3] = v0.w;
        xf4[j][4] = v1.x; xf4[j][5] = v1.y; xf4[j][6] = v1.z; xf4[j][7] = v1.w;
      } else {
        xr[j] = *(const GLB u32x4*)(xb + k0);
      }
      if (nw) wr[j] = *(const GLB u32x4*)(nw + k0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // one memory latency for all of them
  a.ss = 0.f;
#pragma unroll
  for (int j = 0; j < MC; ++j) {
    if (j < a.nc && !xf) {
      xf4[j][0] = bf16lo(xr[j].x); xf4[j][1] = bf16hi(xr[j].x); xf4[j][2] = bf16lo(xr[j].y); xf4[j][3] = bf16hi(xr[j].y);
      xf4[j][4] = bf16lo(xr[j].z); xf4[j][5] = bf16hi(xr[j].z); xf4[j][6] = bf16lo(xr[j].w); xf4[j][7] = bf16hi(xr[j].w);
    }
    float w[8];
    if (j < a.nc && nw) {
      w[0] = bf16lo(wr[j].x); w[1] = bf16hi(wr[j].x); w[2] = bf16lo(wr[j].y); w[3] = bf16hi(wr[j].y);
      w[4] = bf16lo(wr[j].z); w[5] = bf16hi(wr[j].z); w[6] = bf16lo(wr[j].w); w[7] = bf16hi(wr[j].w);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = 1.f;
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (j < a.nc && ok[j]) ? xf4[j][e] : 0.f;
      a.ss = fmaf(x, x, a.ss);
      y[e] = x * w[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const __bf16 h0 = (__bf16)y[2 * e], h1 = (__bf16)y[2 * e + 1];
      a.x[j][e] = __builtin_bit_cast(float, bf16x2{h0, h1});
      a.x[j][4 + e] = __builtin_bit_cast(float, bf16x2{(__bf16)(y[2 * e] - (float)h0), (__bf16)(y[2 * e + 1] - (float)h1)});
    }
  }
  a.ssw = wave_sum(a.ss);
}
__device__ inline void load_act(Act& a, int K, int cw, const GLB float* xf, const GLB uint16_t* xb,
                                const GLB uint16_t* nw) {
  load_act_t<kMaxChunks>(a, K, cw, xf, xb, nw);
}

// Cross-lane butterflies of gfx950: permlane32_swap exchanges the upper half
// of x with the lower half of y, so the sum holds x's pairwise (l, l + 32) sums
// in lanes 0-31 and y's in lanes 32-63; permlane16_swap exchanges the odd
// 16-lane rows of x with the even rows of y, so the sum holds x's (row 0 + row
// 1) in row 0, y's in row 1, x's (row 2 + row 3) in row 2 and y's in row 3.
__device__ __forceinline__ float swap_sum32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_sum16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide sum of NR per-lane accumulators by halving butterflies: NR values
// per lane -> NR/2 (lane halves) -> NR/4 (16-lane rows) -> DPP sums within each
// row, after which row R of the wave holds tile rows r + (NR/4) R, r < NR/4;
// rows < nrows are written to part[].
template <int NR>
__device__ inline void gemv_reduce(const float (&acc)[NR], int nrows, LDS float* part) {
  static_assert(NR == 4 || NR == 8 || NR == 16, "tile rows");
  const int lane = lane_id();
  constexpr int H2 = NR / 2, P = NR / 4;
  float u[H2], v[P];
#pragma unroll
  for (int r = 0; r < H2; ++r) u[r] = swap_sum32(acc[r], acc[r + H2]);
#pragma unroll
  for (int r = 0; r < P; ++r) v[r] = row_sum16(swap_sum16(u[r], u[r + P]));
  const int c = lane & 15, R = lane >> 4;
  float o = v[0];
#pragma unroll
  for (int r = 1; r < P; ++r) o = c == r ? v[r] : o;
  const int row = c + P * R;
  if (c < P && row < nrows) part[row] = o;
}

// Partial dot products of the wave's K range for 'nrows' (<= NR) rows of a
// tile; rows r < n0 come from segment 0, the rest from segment 1 (row r - n0).
// Rows past nrows re-read the last row and chunks outside the wave's range
// re-read chunk 0 (their activations are zero), so every load is issued before
// any is used.  When the wave's share of the tile (NR rows x NC chunks of 16
// bytes per lane) fits in registers, it is read whole, rel() hands the tile's
// LDS pages back to the loaders, and only then pre() waits for the tile's event
// and the activations are loaded: the weights never wait for the event.
// Otherwise (NC == 0: any number of chunks, read chunk by chunk) pre() runs
// first and rel() after the arithmetic.
// 16-byte chunks per lane of a wave's K range (the Act chunk count)
__host__ __device__ inline int gemv_chunks(int K) {
  const int cpw = (K / 8 + kNW - 1) / kNW;
  return (cpw + 63) / 64;
}

// Weight share of one wave: NR rows (rows r < n0 from segment 0, the rest from
// segment 1 as row r - n0) x the 16-byte chunks l, l + 64, ... of the wave's K
// range.  Rows past nrows re-read the last row and chunks outside the range
// re-read chunk 0 (their activations are zero), so every load is issued before
// any is used.
struct GemvGeom {
  int nch, cpw, base, rb, n0, nrows;
  __device__ GemvGeom(const GemvIn& gi, int cw)
      : nch(gi.K / 8), cpw((gi.K / 8 + kNW - 1) / kNW), base(cw * ((gi.K / 8 + kNW - 1) / kNW)), rb(gi.K * 2),
        n0(gi.n0), nrows(gi.nrows) {}
};
template <int NR, class Src>
__device__ __forceinline__ void gemv_load_chunk(const Src& src, const GemvGeom& g, int j, uint4* wv) {
  const int ch = lane_id() + 64 * j;
  const int cb = (ch < g.cpw && g.base + ch < g.nch ? g.base + ch : 0) * 16;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rc = r < g.nrows ? r : g.nrows - 1;
    const int seg = rc < g.n0 ? 0 : 1;
    const int rr = rc < g.n0 ? rc : rc - g.n0;
    wv[r] = src.ld16(seg, rr * g.rb + cb);
  }
}
template <int NR>
__device__ __forceinline__ void gemv_fma_chunk(const Act& a, int j, const uint4* wv, float (&acc)[NR]) {
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint4 u = wv[r];
    const bf16x2 w0 = __builtin_bit_cast(bf16x2, u.x), w1 = __builtin_bit_cast(bf16x2, u.y);
    const bf16x2 w2 = __builtin_bit_cast(bf16x2, u.z), w3 = __builtin_bit_cast(bf16x2, u.w);
    float s = acc[r];
    s = __builtin_amdgcn_fdot2_f32_bf16(w0, act_pair(a, j, 0), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w1, act_pair(a, j, 1), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w2, act_pair(a, j, 2), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w3, act_pair(a, j, 3), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w0, act_pair(a, j, 4), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w1, act_pair(a, j, 5), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w2, act_pair(a, j, 6), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(w3, act_pair(a, j, 7), s, false);
    acc[r] = s;
  }
}
// the whole share (NR x NC <= 16 registers of 16 bytes) into wv
template <int NR, int NC, class Src>
__device__ __forceinline__ void gemv_pull(const Src& src, const GemvGeom& g, uint4 (&wv)[16]) {
#pragma unroll
  for (int j = 0; j < NC; ++j) gemv_load_chunk<NR>(src, g, j, &wv[j * NR]);
}
template <int NR, int NC>
__device__ __forceinline__ void gemv_finish(const Act& a, const uint4 (&wv)[16], int nrows, LDS float* part) {
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < NC; ++j) gemv_fma_chunk<NR>(a, j, &wv[j * NR], acc);
  gemv_reduce<NR>(acc, nrows, part);
}
// two rows of up to kMaxChunks chunks (the whole share in 2 x NC registers),
// reduced as a 4-row block whose last two rows are zero
template <int NC>
__device__ __forceinline__ void gemv_finish2(const Act& a, const uint4 (&wv)[16], int nrows, LDS float* part) {
  float acc2[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NC; ++j) gemv_fma_chunk<2>(a, j, &wv[j * 2], acc2);
  const float acc[4] = {acc2[0], acc2[1], 0.f, 0.f};
  gemv_reduce<4>(acc, nrows, part);
}
// any K, 4 rows, chunk by chunk (the activations are already loaded)
template <class Src>
__device__ inline void gemv_chunked(const Src& src, const Act& a, const GemvGeom& g, LDS float* part) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    if (j < a.nc) {
      uint4 wv[4];
      gemv_load_chunk<4>(src, g, j, wv);
      __builtin_amdgcn_sched_barrier(0);
      gemv_fma_chunk<4>(a, j, wv, acc);
    }
  }
  gemv_reduce<4>(acc, g.nrows, part);
}

// One GEMV tile for one compute wave.  When its weight share fits in registers
// (the tile shapes below), the share is read whole from LDS, rel() hands the
// tile's pages back to the loaders, and only then pre() waits for the tile's
// event and says whether the activations must be loaded (false when an earlier
// tile of the same op left them in a): the weights never wait for the event.
// Otherwise pre() runs first and rel() after the arithmetic.  The activation
// load has one call site, so it is inlined once.
template <int POL = 0, class Src, class Rel, class Pre>
__device__ inline void gemv_rows(const Src& src, Act& a, const GemvIn& gi, int cw, LDS float* part, const Rel& rel,
                                 const Pre& pre) {
  const GemvGeom g(gi, cw);
  const int nc = gemv_chunks(gi.K);
  const int shape = nc == 1 ? 0 : nc == 2 ? 1 : nc <= 4 ? 2 : (nc <= kMaxChunks && g.nrows <= 2) ? 4 : 3;
  uint4 wv[16];
  if (shape == 0)
    gemv_pull<16, 1>(src, g, wv);
  else if (shape == 1)
    gemv_pull<8, 2>(src, g, wv);
  else if (shape == 2)
    gemv_pull<4, 4>(src, g, wv);
  else if (shape == 4)
    gemv_pull<2, kMaxChunks>(src, g, wv);
  // keep every LDS read of the share in flight at once: without this boundary
  // the scheduler interleaves each read with the previous row's FMAs and waits
  // for it, paying the LDS latency once per row
  __builtin_amdgcn_sched_barrier(0);
  if (shape != 3) rel();
  if (pre()) load_act_t<kMaxChunks, POL>(a, gi.K, cw, gi.xf, gi.xb, gi.nw);
  if (shape == 0)
    gemv_finish<16, 1>(a, wv, g.nrows, part);
  else if (shape == 1)
    gemv_finish<8, 2>(a, wv, g.nrows, part);
  else if (shape == 2)
    gemv_finish<4, 4>(a, wv, g.nrows, part);
  else if (shape == 4)
    gemv_finish2<kMaxChunks>(a, wv, g.nrows, part);
  else {
    gemv_chunked(src, a, g, part);
    rel();
  }
}


// Tile shapes, by 16-byte chunks per lane nc = ceil(K / 2048): nc = 1 -> up to
// 16 rows, nc = 2 -> up to 8, nc = 3..4 -> up to 4 (the wave's share, at most
// 16 x 16 bytes per lane, is read whole); larger K -> up to 2 rows read whole,
// or up to 4 rows chunk by chunk (their pages held until the arithmetic ends).
// Few shapes keep the interpreter's code within the instruction cache; the plan
// builder rejects tiles with more rows (gemv_max_rows).
__host__ __device__ inline int gemv_max_rows(int K) {
  const int nc = (K + 2047) / 2048;
  return nc <= 1 ? 16 : nc == 2 ? 8 : 4;
}

__device__ __forceinline__ int op_sum_rows(int op, const Consts& c) {
  return op == OpGateUp || op == OpOproj ? c.ssg_f : c.ssg_a;
}
__device__ inline GemvIn gemv_input(const Meta& m, const Consts& c) {
  GemvIn g;
  g.xf = nullptr;
  g.xb = nullptr;
  g.nw = nullptr;
  g.emb = nullptr;
  g.tok = nullptr;
  g.xs = nullptr;
  g.ssc = nullptr;
  g.ssg = op_sum_rows(m.w(WOpcode), c);
  g.norm = 0;
  const bool split = c.B > 1;  // batch > 1: inputs in pre-split form (act_split)
  const int op = m.w(WOpcode);
  switch (op) {
    case OpQkv:
      g.K = c.H;
      g.norm = 1;
      if (m.q(QkvX)) {
        if (split) {
          g.xs = (const GLB char*)m.q(QkvPrep);
          g.ssc = (const GLB float*)m.q(QkvSs);
        } else {
          g.xf = (const GLB float*)m.q(QkvX);
          g.nw = (const GLB uint16_t*)m.q(QkvNorm);
        }
      } else {
        g.nw = (const GLB uint16_t*)m.q(QkvNorm);
        g.emb = (const GLB uint16_t*)m.q(QkvEmbed);
        g.tok = (const GLB int*)m.q(QkvTokens);
        if (c.B == 1) g.xb = g.emb + (size_t)token0(m.q(QkvTokens), c.V) * c.H;
      }
      g.n0 = g.nrows = m.w(WPay + 1);
      break;
    case OpOproj:
      g.K = c.nq * c.hd;
      if (split)
        g.xs = (const GLB char*)m.q(OIn);
      else
        g.xf = (const GLB float*)m.q(OIn);
      g.n0 = g.nrows = m.w(WPay + 1);
      break;
    case OpGateUp:
      g.K = c.H;
      g.norm = 1;
      if (split) {
        g.xs = (const GLB char*)m.q(GuPrep);
        g.ssc = (const GLB float*)m.q(GuSs);
      } else {
        g.nw = (const GLB uint16_t*)m.q(GuNorm);
        g.xf = (const GLB float*)m.q(GuIn);
      }
      g.n0 = m.w(WPay + 1);
      g.nrows = 2 * m.w(WPay + 1);
      break;
    case OpDown:
      g.K = c.F;
      if (split)
        g.xs = (const GLB char*)m.q(DnIn);
      else
        g.xf = (const GLB float*)m.q(DnIn);
      g.n0 = g.nrows = m.w(WPay + 1);
      break;
    default:  // OpLmHead
      g.K = c.H;
      g.norm = 1;
      if (split) {
        g.xs = (const GLB char*)m.q(LmPrep);
        g.ssc = (const GLB float*)m.q(LmSs);
      } else {
        g.nw = (const GLB uint16_t*)m.q(LmNorm);
        g.xf = (const GLB float*)m.q(LmIn);
      }
      g.n0 = g.nrows = m.w(WPay + 1);
      break;
  }
  return g;
}

// Residual input of a GEMV tile's rows (O projection: the residual stream or,
// in layer 0, the embedding row; down projection: the post-attention stream),
// one value per lane < nrows; loaded ahead of the epilogue.
template <int POL = 0>
__device__ inline float gemv_residual(const Meta& m, const Consts& c) {
  const int lane = lane_id();
  const int op = m.w(WOpcode);
  const int row0 = m.w(WPay), nr = m.w(WPay + 1);
  const int rr = row0 + (lane < nr ? lane : 0);
  if (op == OpOproj)
    return m.q(OX) ? CohT<POL>((const GLB float*)m.q(OX)).f1(rr * 4)
                    : bf16f(((const GLB uint16_t*)m.q(OEmbed))[(size_t)token0(m.q(OTokens), c.V) * c.H + rr]);
  if (op == OpDown) return CohT<POL>((const GLB float*)m.q(DnRes)).f1(rr * 4);
  return 0.f;
}

// Epilogue of a GEMV tile, run by one wave once every compute wave's partials
// (part[w][r]) and partial sums of squares (ssp[w]) are in LDS.
__device__ inline void gemv_epilogue(const Meta& m, const Consts& c,
                                     const LDS float (*part)[kMaxRows], const LDS float* ssp, float res) {
  const int lane = lane_id();
  const int op = m.w(WOpcode);
  const GemvIn g = gemv_input(m, c);
  float scale = 1.f;
  if (g.norm) {
    float ss = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) ss += ssp[w];
    scale = 1.f / sqrtf(ss / (float)g.K + c.eps);
  }
  float v = 0.f;
  if (lane < g.nrows) {
#pragma unroll
    for (int w = 0; w < kNW; ++w) v += part[w][lane];
    v *= scale;
  }
  const int row0 = m.w(WPay), nr = m.w(WPay + 1);
  switch (op) {
    case OpQkv:
      if (lane < nr) st_agent((GLB float*)m.q(QkvOut) + (size_t)m.w(WGx) * c.RPG + row0 + lane, v);
      break;
    case OpOproj:
      if (lane < nr) st_agent((GLB float*)m.q(OOut) + row0 + lane, res + v);
      break;
    case OpGateUp: {
      float u = __shfl(v, lane + nr, 64);  // up row j sits at tile row nr + j
      if (lane < nr) st_agent((GLB float*)m.q(GuOut) + row0 + lane, v / (1.f + __expf(-v)) * u);
      break;
    }
    case OpDown:
      if (lane < nr) st_agent((GLB float*)m.q(DnOut) + row0 + lane, res + v);
      break;
    case OpLmHead: {
      if (lane < nr) ((GLB float*)m.q(LmLogits))[row0 + lane] = v;
      // tile max, lowest row on ties
      float bv = lane < nr ? v : -INFINITY;
      int bi = lane < nr ? row0 + lane : 0x7FFFFFFF;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        float ov = __shfl_xor(bv, m, 64);
        int oi = __shfl_xor(bi, m, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == 0) {
        GLB float* mx = (GLB float*)m.q(LmMax) + 2 * (size_t)m.w(WGx);
        st_agent(mx, bv);
        st_agent((GLB int*)mx + 1, bi);
      }
      break;
    }
    default:
      break;
  }
}

__device__ __forceinline__ bool amax_better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// ---- batched GEMV (B <= 16 sequences) on the matrix cores ----------------------
// A tile is up to 16 weight rows x K; each compute wave takes a quarter of K in
// steps of 32 and accumulates one v_mfma_f32_16x16x32_bf16 block: A = the 16
// weight rows (lane l: row l % 16, k = 8 (l / 16) .. +7, one 16-byte LDS read),
// B = the sequences' activations (lane l: sequence l % 16, the same 8 k), C =
// 16 rows x 16 sequences (lane l: sequence l % 16, rows 4 (l / 16) .. +3).  The
// fp32 activations (times the RMSNorm weight) enter as two bf16 parts, hi =
// bf16(x) and lo = bf16(x - hi), one MFMA each: the weight x activation
// products keep about 16 bits of the activation, as the fp32 path does to
// within rounding.  The producers store the activations already split
// (act_split), so a k-step is two 16-byte loads straight into the MFMA
// operands, and the fused norm's sums of squares come with the residual
// (gemv_sumsq_mb); only layer 0's QKV, whose input is the token's bf16
// embedding row, splits and squares in the tile.  Rows
// past nrows re-read the last row; sequences past B and chunks past the
// wave's range read valid addresses and are zeroed.
// kpart / nparts: the tile's K range is cut into nparts equal parts (K / 8 a
// multiple of nparts) and this call runs part kpart; a part after the first
// adds its sums to the ones already in part / ssp (the earlier parts', written
// by this wave or, in the megakernel, by the owning group's wave cw), so the
// result is (part 0 + part 1) in that order wherever the tile runs.
template <bool EMB, int POL, class Src, class Rel>
__device__ inline void gemv_tile_mb(const Src& src, const GemvIn& gi, int B, int V, int cw, LDS float* part,
                                    LDS float* ssp, const Rel& rel, int kpart, int nparts) {
  const int lane = lane_id();
  const int K = gi.K, nch = K / 8 / nparts, c0 = kpart * nch, cpw = (nch + kNW - 1) / kNW, base = c0 + cw * cpw;
  const int nks = (cpw + 3) / 4;  // k-steps of 4 chunks
  const int r = lane & 15, q = lane >> 4;
  const int rc = r < gi.nrows ? r : gi.nrows - 1;
  const int seg = rc < gi.n0 ? 0 : 1, rr = rc < gi.n0 ? rc : rc - gi.n0;
  const int arow = rr * K * 2;
  const int b = lane & 15;
  const bool bok = b < B;
  const int bb = bok ? b : 0;
  const GLB uint16_t* xb = nullptr;
  if (EMB) xb = gi.emb + (size_t)token_of(gi.tok, bb, V) * K;
  const CohT<POL> cx(EMB ? (const GLB void*)gi.emb : (const GLB void*)gi.xs);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  constexpr int NB = 4;  // k-steps whose loads are issued together
  for (int ks0 = 0; ks0 < nks; ks0 += NB) {
    u32x4 A[NB], xr[NB], wn[NB], xh[NB], xl[NB];
    bool ok[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int ks = ks0 + u, ch = ks * 4 + q;
      ok[u] = ks < nks && ch < cpw && base + ch < c0 + nch;
      const int chunk = ok[u] ? base + ch : 0, kk = chunk * 8;
      const uint4 w = src.ld16(seg, arow + kk * 2);
      A[u] = u32x4{w.x, w.y, w.z, w.w};
      if (EMB) {
        xr[u] = *(const GLB u32x4*)(xb + kk);
        if (gi.nw) wn[u] = *(const GLB u32x4*)(gi.nw + kk);
      } else {
        const uint32_t xo = (uint32_t)((chunk * B + bb) * 32);  // split_off(bb, kk, B)
        xh[u] = cx.u4(xo);
        xl[u] = cx.u4(xo + 16);

      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool live = ok[u] && bok;
      const bf16x8 av = __builtin_bit_cast(bf16x8, A[u]);
      if (!EMB) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, live ? xh[u] : z), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, live ? xl[u] : z), acc, 0, 0, 0);
        continue;
      }
      float v[8];
      v[0] = bf16lo(xr[u].x); v[1] = bf16hi(xr[u].x); v[2] = bf16lo(xr[u].y); v[3] = bf16hi(xr[u].y);
      v[4] = bf16lo(xr[u].z); v[5] = bf16hi(xr[u].z); v[6] = bf16lo(xr[u].w); v[7] = bf16hi(xr[u].w);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[e] = live ? v[e] : 0.f;
        ss = fmaf(v[e], v[e], ss);
      }
      if (gi.nw) {
        v[0] *= bf16lo(wn[u].x); v[1] *= bf16hi(wn[u].x); v[2] *= bf16lo(wn[u].y); v[3] *= bf16hi(wn[u].y);
        v[4] *= bf16lo(wn[u].z); v[5] *= bf16hi(wn[u].z); v[6] *= bf16lo(wn[u].w); v[7] *= bf16hi(wn[u].w);
      }
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 h = (__bf16)v[e];
        hi[e] = h;
        lo[e] = (__bf16)(v[e] - (float)h);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hi, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, lo, acc, 0, 0, 0);
    }
  }
  rel();
  // sequence b's sum of squares over the wave's range: lanes b, b+16, b+32, b+48
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (kpart == 0) {
    if (lane < kMB) ssp[lane] = ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(4 * q + i) * kMB + b] = acc[i];
  } else {
    if (lane < kMB) ssp[lane] = ssp[lane] + ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(4 * q + i) * kMB + b] = part[(4 * q + i) * kMB + b] + acc[i];
  }
}

template <int POL = 0, class Src, class Rel>
__device__ inline void gemv_rows_mb(const Src& src, const GemvIn& gi, int B, int V, int cw, LDS float* part,
                                    LDS float* ssp, const Rel& rel, int kpart = 0, int nparts = 1) {
  if (gi.xs)
    gemv_tile_mb<false, POL>(src, gi, B, V, cw, part, ssp, rel, kpart, nparts);
  else
    gemv_tile_mb<true, POL>(src, gi, B, V, cw, part, ssp, rel, kpart, nparts);
}

// Batched QKV, O-projection and down tiles run their K range in two halves:
// in the megakernel the instruction's own compute group takes the first half
// and the other group, otherwise idle through these ops (at most one tile of
// them per compute unit), the second; the layer-by-layer kernel runs both
// halves in turn.  The sums are added in the same order either way.
__device__ __forceinline__ bool gemv_k_halves(int op, const Consts& c) {
  if (c.B <= 1 || c.glm) return false;
  const int K = op == OpQkv ? c.H : op == OpOproj ? c.nq * c.hd : op == OpDown ? c.F : 0;
  return K > 0 && K % 16 == 0;
}

// Batched O-projection, gate/up and down tiles whose output rows are whole
// 8-row chunks (row0 and the row count multiples of 8) run a chunk-wise
// epilogue: lane (chunk l / 16, sequence l % 16) owns the chunk's 8 outputs, so
// the residual, the stored residual stream, the norm weight and the split
// copy move as 16-byte vectors.  Other tiles (row counts not a multiple of 8)
// keep the element-wise one.
__device__ __forceinline__ bool mb_chunk_tile(const Meta& m, const Consts& c) {
  const int op = m.w(WOpcode);
  // (O and down keep their sums of squares per chunk only when every tile of
  // the op has whole chunks)
  return (op == OpGateUp || ((op == OpOproj || op == OpDown) && op_sum_rows(op, c) == 8)) && (m.w(WPay) & 7) == 0 &&
         (m.w(WPay + 1) & 7) == 0;
}
struct ResMB {
  f32x4 r0, r1;  // chunk-wise: the chunk's 8 residuals; element-wise: r0 = the lane's 4
  float ss;      // pre-split input with a fused norm: sequence lane % 16's sum of squares
};
// Residual inputs of the batched epilogue, loaded before the tile's partial
// sums are in (element-wise: lane l owns index idx = l + 64 j, row idx / 16,
// sequence idx % 16 = l % 16).
template <int POL = 0>
__device__ inline ResMB gemv_residual_mb(const Meta& m, const Consts& c) {
  const int lane = lane_id();
  const int op = m.w(WOpcode);
  ResMB r;
  r.r0 = f32x4{0.f, 0.f, 0.f, 0.f};
  r.r1 = r.r0;
  r.ss = 0.f;
  if (op != OpOproj && op != OpDown) return r;
  const int row0 = m.w(WPay), nr = m.w(WPay + 1);
  const int b = lane & 15, bb = b < c.B ? b : 0;
  if (mb_chunk_tile(m, c)) {
    const int cl = (lane >> 4) < (nr >> 3) ? (lane >> 4) : 0;
    const int k = row0 + 8 * cl;
    if (op == OpOproj && !m.q(OX)) {
      const u32x4 e = *(const GLB u32x4*)((const GLB uint16_t*)m.q(OEmbed) +
                                          (size_t)token_of((const GLB int*)m.q(OTokens), bb, c.V) * c.H + k);
      r.r0 = f32x4{bf16lo(e.x), bf16hi(e.x), bf16lo(e.y), bf16hi(e.y)};
      r.r1 = f32x4{bf16lo(e.z), bf16hi(e.z), bf16lo(e.w), bf16hi(e.w)};
    } else {
      const CohT<POL> cx((const GLB float*)m.q(op == OpOproj ? OX : DnRes));
      const uint32_t o = (uint32_t)act_ix(bb, k, c.B) * 4;
      r.r0 = cx.f4(o);
      r.r1 = cx.f4(o + 16);
    }
    return r;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (lane + 64 * j) >> 4;
    const int rr = row0 + (row < nr ? row : 0);
    if (op == OpOproj) {
      r.r0[j] = m.q(OX) ? CohT<POL>((const GLB float*)m.q(OX)).f1((uint32_t)act_ix(bb, rr, c.B) * 4)
                        : bf16f(((const GLB uint16_t*)m.q(OEmbed))[(size_t)token_of((const GLB int*)m.q(OTokens), bb,
                                                                                     c.V) * c.H + rr]);
    } else {
      r.r0[j] = CohT<POL>((const GLB float*)m.q(DnRes)).f1((uint32_t)act_ix(bb, rr, c.B) * 4);
    }
  }
  return r;
}

// Batch > 1, a fused norm over a pre-split input: the input's sum of squares
// for sequence lane % 16, from the producers' sums over groups of ssg rows
// ([b][H / ssg]).  Lane (b, p = lane / 16) adds the p-th quarter in order,
// then the quarters are added (fixed order, the same in every kernel).
// Returns 0 for other ops.
template <int POL = 0>
__device__ inline float gemv_sumsq_mb(const Meta& m, const Consts& c) {
  const GemvIn g = gemv_input(m, c);
  if (!g.norm || !g.xs) return 0.f;
  const int lane = lane_id();
  const int b = lane & 15, bb = b < c.B ? b : 0, p = lane >> 4;
  const int n = c.H / g.ssg, per = (n + 3) / 4;  // sums per sequence, per lane
  const CohT<POL> cs((const GLB void*)g.ssc);
  float t = 0.f;
  const int i0 = p * per;
  if (n % 16 == 0) {  // quarters of whole 16-byte runs, eight loads in flight
    for (int i = 0; i < per; i += 32) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = i + 4 * u < per ? cs.f4((uint32_t)(bb * n + i0 + i + 4 * u) * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < 8; ++u) t += ((v[u].x + v[u].y) + (v[u].z + v[u].w));
    }
  } else {
    for (int i = 0; i < per && i0 + i < n; ++i) t += cs.f1((uint32_t)(bb * n + i0 + i) * 4);
  }
  t += __shfl_xor(t, 16, 64);
  t += __shfl_xor(t, 32, 64);
  return t;
}

// 16 bytes from 8 floats' bf16 high parts (hi) or low parts (lo = bf16(v - h))
__device__ __forceinline__ void split8(const float* v, u32x4& hi, u32x4& lo) {
  bf16x8 h, l;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 t = (__bf16)v[e];
    h[e] = t;
    l[e] = (__bf16)(v[e] - (float)t);
  }
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, l);
}

// Epilogue of a batched GEMV tile: part[w * 256 + row * 16 + b] are wave w's
// partial sums, ssp[w * 16 + b] its sums of squares of sequence b.
__device__ inline void gemv_epilogue_mb(const Meta& m, const Consts& c, const LDS float* part, const LDS float* ssp,
                                        ResMB rs) {
  const f32x4 res = rs.r0;
  const int lane = lane_id();
  const int op = m.w(WOpcode);
  const GemvIn g = gemv_input(m, c);
  const int b = lane & 15;
  const bool bok = b < c.B;
  float scale = 1.f;
  if (g.norm) {
    float ss = 0.f;
    if (g.xs) {
      ss = rs.ss;  // from the producers' sums (gemv_sumsq_mb)
    } else {
#pragma unroll
      for (int w = 0; w < kNW; ++w) ss += ssp[w * kMB + b];
    }
    scale = 1.f / sqrtf(ss / (float)g.K + c.eps);
  }
  const int row0 = m.w(WPay), nr = m.w(WPay + 1);
  auto val = [&](int row) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) v += part[w * kMB * kMB + row * kMB + b];
    return v * scale;
  };
  if (mb_chunk_tile(m, c)) {
    // lane (chunk cl, sequence b); stores through buffer resources with
    // sc1 (st_agent16), everything 16 bytes per lane
    const int cl = lane >> 4;
    if (cl >= (nr >> 3) || !bok) return;
    const int r0 = 8 * cl, k = row0 + r0;
    const uint32_t so = split_off(b, k, c.B);
    float x[8];
    if (op == OpGateUp) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gt = val(r0 + e), up = val(nr + r0 + e);  // up row j sits at tile row nr + j
        x[e] = gt / (1.f + __expf(-gt)) * up;
      }
      u32x4 hi, lo;
      split8(x, hi, lo);
      st_agent16((const GLB void*)m.q(GuOut), so, __builtin_bit_cast(f32x4, hi));
      st_agent16((const GLB void*)m.q(GuOut), so + 16, __builtin_bit_cast(f32x4, lo));
      return;
    }
    // O projection / down: x = residual + W a, stored as is; x times the next
    // op's norm weight, split; the chunk's sum of squares of x
    const u32x4 wq = *(const GLB u32x4*)((const GLB uint16_t*)m.q(op == OpOproj ? OPrepW : DnPrepW) + k);
    const float w8[8] = {bf16lo(wq.x), bf16hi(wq.x), bf16lo(wq.y), bf16hi(wq.y),
                         bf16lo(wq.z), bf16hi(wq.z), bf16lo(wq.w), bf16hi(wq.w)};
    const float rv[8] = {rs.r0.x, rs.r0.y, rs.r0.z, rs.r0.w, rs.r1.x, rs.r1.y, rs.r1.z, rs.r1.w};
    float y[8], sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = rv[e] + val(r0 + e);
      y[e] = x[e] * w8[e];
      sq = fmaf(x[e], x[e], sq);
    }
    const uint32_t xo = (uint32_t)act_ix(b, k, c.B) * 4;
    const GLB void* xout = (const GLB void*)m.q(op == OpOproj ? OOut : DnOut);
    st_agent16(xout, xo, f32x4{x[0], x[1], x[2], x[3]});
    st_agent16(xout, xo + 16, f32x4{x[4], x[5], x[6], x[7]});
    u32x4 hi, lo;
    split8(y, hi, lo);
    const GLB void* xs = (const GLB void*)m.q(op == OpOproj ? OPrep : DnPrep);
    st_agent16(xs, so, __builtin_bit_cast(f32x4, hi));
    st_agent16(xs, so + 16, __builtin_bit_cast(f32x4, lo));
    // one sum per chunk (the row counts are multiples of 8, so the sums are
    // kept per chunk: [B][H / 8])
    st_agent((GLB float*)m.q(op == OpOproj ? OSs : DnSs) + (size_t)b * (c.H / 8) + (k >> 3), sq);
    return;
  }
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  // O projection and down: the residual stream x is stored as is, and again
  // split and times the next op's RMSNorm weight (gate/up's; the next layer's
  // QKV or the LM head's) with its sums of squares over groups of rows, which
  // the next op's tiles add instead of squaring x themselves.
  const bool resid = op == OpOproj || op == OpDown;
  const GLB uint16_t* wnext = resid ? (const GLB uint16_t*)m.q(op == OpOproj ? OPrepW : DnPrepW) : nullptr;
  const GLB void* xsplit = resid ? (const GLB void*)m.q(op == OpOproj ? OPrep : DnPrep) : nullptr;
  float sq[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (lane + 64 * j) >> 4;
    const bool live = bok && row < nr;
    sq[j] = 0.f;
    switch (op) {
      case OpQkv:
        if (live) st_agent((GLB float*)m.q(QkvOut) + ((size_t)b * c.nkv + m.w(WGx)) * c.RPG + row0 + row, val(row));
        break;
      case OpOproj:
      case OpDown:
        if (live) {
          const float x = res[j] + val(row);
          st_agent((GLB float*)m.q(op == OpOproj ? OOut : DnOut) + act_ix(b, row0 + row, c.B), x);
          st_split(xsplit, b, row0 + row, c.B, x * bf16f(wnext[row0 + row]));
          sq[j] = x * x;
        }
        break;
      case OpGateUp:
        if (live) {
          const float gt = val(row), up = val(nr + row);  // up row j sits at tile row nr + j
          st_split((const GLB void*)m.q(GuOut), b, row0 + row, c.B, gt / (1.f + __expf(-gt)) * up);
        }
        break;
      case OpLmHead:
        if (live) {
          const float v = val(row);
          ((GLB float*)m.q(LmLogits))[(size_t)b * c.V + row0 + row] = v;
          if (amax_better(v, row0 + row, bv, bi)) {
            bv = v;
            bi = row0 + row;
          }
        }
        break;
      default:
        break;
    }
  }
  if (resid) {
    // sums of squares of x over groups of g rows (g divides the tile rows, so
    // row0 starts a group), stored [b][H / g].  Lane
    // (b, q = lane / 16) holds rows q + 4 j; lanes b, b+16, b+32, b+48 hold
    // sequence b's rows.
    const int g = op_sum_rows(op, c);
    GLB float* ssc = (GLB float*)m.q(op == OpOproj ? OSs : DnSs);
    const int q = lane >> 4;
    auto put = [&](int grp, float v) {  // grp: the group's first row within the tile
      st_agent(ssc + (size_t)b * (c.H / g) + (row0 + grp) / g, v);
    };
    if (g == 8) {
      float p0 = sq[0] + sq[1], p1 = sq[2] + sq[3];  // rows 0..7, 8..15
      p0 += __shfl_xor(p0, 16, 64);
      p1 += __shfl_xor(p1, 16, 64);
      p0 += __shfl_xor(p0, 32, 64);
      p1 += __shfl_xor(p1, 32, 64);
      if (q == 0 && bok) {
        put(0, p0);
        if (nr > 8) put(8, p1);
      }
    } else if (g == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // rows 4 j .. 4 j + 3
        float t = sq[j];
        t += __shfl_xor(t, 16, 64);
        t += __shfl_xor(t, 32, 64);
        if (q == 0 && bok && 4 * j < nr) put(4 * j, t);
      }
    } else if (g == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // rows q + 4 j and q + 1 + 4 j, q even
        const float t = sq[j] + __shfl_xor(sq[j], 16, 64);
        if ((q & 1) == 0 && bok && q + 4 * j < nr) put(q + 4 * j, t);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (bok && q + 4 * j < nr) put(q + 4 * j, sq[j]);
    }
  }
  if (op == OpLmHead) {
    // lanes b, b+16, b+32, b+48 hold sequence b's rows: the tile's (max, lowest index)
#pragma unroll
    for (int msk = 16; msk <= 32; msk <<= 1) {
      const float ov = __shfl_xor(bv, msk, 64);
      const int oi = __shfl_xor(bi, msk, 64);
      if (amax_better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane < kMB && bok) {
      GLB float* mx = (GLB float*)m.q(LmMax) + 2 * ((size_t)b * c.T_v + m.w(WGx));
      st_agent(mx, bv);
      st_agent((GLB int*)mx + 1, bi);
    }
  }
}

__device__ __forceinline__ bool is_gemv(int op) {
  return op == OpQkv || op == OpOproj || op == OpGateUp || op == OpDown || op == OpLmHead;
}

// ---- attention -----------------------------------------------------------------
// One wave per query head of the kv group: RoPE (and Qwen3's q/k RMSNorm), the
// new K/V row (written to the cache by wave 0 of the split that holds it),
// scores over the split's positions, and the partial (max, sum, weighted V).
// Every global input is loaded in one batch up front; the RoPE partner of
// element d (d +- head_dim/2) is in the same lane for head_dim 128 and in
// lane ^ 32 for head_dim 64.
// The attention task's prologue, the same for every attention kernel: the
// wave's q head (cw; head 0 for waves past the group's heads) rotated into
// scr[0, HD), the new K/V row (when the split holds it) as bf16 in scr after
// it, written to the cache by the writer wave.  Returns the task's positions.
struct AttnTask {
  int b, g, s, lo, hi, pos, nk;
  bool has_new, active;
};
template <int HD, int POL = 0>
__device__ inline AttnTask attn_prologue(const Meta& mt, const Consts& c, int cw, LDS float* scr, bool writer) {
  const int lane = lane_id();
  const int b = mt.w(WGx), g = mt.w(WGy), s = mt.w(WGz);
  const int lo = mt.w(WPay), hi = mt.w(WPay + 1), pos = mt.w(WPay + 2);
  int nk = (hi < pos ? hi : pos) - lo;
  if (nk < 0) nk = 0;
  const bool has_new = pos >= lo && pos < hi;
  const bool active = cw < c.hpg;
  constexpr int HALF = HD / 2;
  constexpr int PER = HD / 64;  // head elements per lane: d = lane + 64 k
  const CohT<POL> cq((const GLB float*)mt.q(AttnQkv) + ((size_t)b * c.nkv + g) * c.RPG);
  const GLB float* rope = (const GLB float*)mt.q(AttnRope) + (size_t)b * HD;  // (cos, sin) pairs
  const GLB uint16_t* qn = c.qk_norm ? (const GLB uint16_t*)mt.q(AttnQn) : nullptr;
  const GLB uint16_t* knw = c.qk_norm ? (const GLB uint16_t*)mt.q(AttnKn) : nullptr;
  LDS float* qs = scr;                                   // rotated q, HD floats
  LDS uint16_t* kn = (LDS uint16_t*)(scr + HD);          // new k row as the cache holds it (bf16), HD
  LDS uint16_t* vn = (LDS uint16_t*)(scr + 2 * HD);      // new v row (bf16), HD

  // ---- one batch of global loads
  float qv[PER], kv[PER], vv[PER], cs[PER], sn[PER], wq[PER], wk[PER];
  const int qh = active ? cw : 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int d = lane + 64 * k;
    const int ii = d < HALF ? d : d - HALF;
    qv[k] = cq.f1((uint32_t)(qh * HD + d) * 4);
    kv[k] = cq.f1((uint32_t)(c.hpg * HD + d) * 4);
    vv[k] = cq.f1((uint32_t)((c.hpg + 1) * HD + d) * 4);
    cs[k] = rope[2 * ii];
    sn[k] = rope[2 * ii + 1];
    wq[k] = qn ? bf16f(qn[d]) : 1.f;
    wk[k] = knw ? bf16f(knw[d]) : 1.f;
  }
  // ---- per-head RMSNorm (Qwen3) and rotate-half RoPE, in registers
  auto norm_rot = [&](float* v, const float* w, bool do_norm) {
    if (do_norm) {
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k) ss = fmaf(v[k], v[k], ss);
      ss = wave_sum(ss);
      const float inv = 1.f / sqrtf(ss / (float)HD + c.eps);
#pragma unroll
      for (int k = 0; k < PER; ++k) v[k] = v[k] * inv * w[k];
    }
    float partner[PER];
    if (PER == 1) {
      partner[0] = __shfl_xor(v[0], 32, 64);
    } else {
      partner[0] = v[PER - 1];
      partner[PER - 1] = v[0];
    }
    float r[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      r[k] = d < HALF ? v[k] * cs[k] - partner[k] * sn[k] : v[k] * cs[k] + partner[k] * sn[k];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = r[k];
  };
  norm_rot(qv, wq, c.qk_norm != 0);
#pragma unroll
  for (int k = 0; k < PER; ++k) qs[lane + 64 * k] = qv[k];
  if (has_new) {
    norm_rot(kv, wk, c.qk_norm != 0);
    uint16_t kb[PER], vb[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      kb[k] = f2bf(kv[k]);
      vb[k] = f2bf(vv[k]);
      kn[lane + 64 * k] = kb[k];
      vn[lane + 64 * k] = vb[k];
    }
    if (writer) {
      const size_t row = (((size_t)b * c.nkv + g) * c.cap + pos) * HD;
      GLB uint16_t* K = (GLB uint16_t*)mt.q(AttnK) + row;
      GLB uint16_t* Vv = (GLB uint16_t*)mt.q(AttnV) + row;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        K[lane + 64 * k] = kb[k];
        Vv[lane + 64 * k] = vb[k];
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  return AttnTask{b, g, s, lo, hi, pos, nk, has_new, active};
}

template <int HD, int POL = 0, class Src>
__device__ inline void attn_wave(const Src& src, const Meta& mt, const Consts& c, int cw,
                                 LDS float* scr, bool writer, unsigned long long* tr = nullptr) {
  const int lane = lane_id();
  const AttnTask at = attn_prologue<HD, POL>(mt, c, cw, scr, writer);
  const int b = at.b, g = at.g, s = at.s, nk = at.nk;
  const bool has_new = at.has_new, active = at.active;
  LDS float* qs = scr;                               // rotated q, HD floats
  LDS uint16_t* kn = (LDS uint16_t*)(scr + HD);      // new k row (bf16), HD
  LDS uint16_t* vn = (LDS uint16_t*)(scr + 2 * HD);  // new v row (bf16), HD
  constexpr int PER = HD / 64;
  if (tr && lane == 0) tr[6] = now_ticks();
  if (!active) return;
  const int n = nk + (has_new ? 1 : 0);
  GLB float* outp = (GLB float*)mt.q(AttnOut) + ((((size_t)b * c.nkv + g) * c.S + s) * c.hpg + cw) * (HD + 2);
  if (n == 0) {
    if (lane == 0) {
      st_agent(outp, -INFINITY);
      st_agent(outp + 1, 0.f);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) st_agent(outp + 2 + lane + 64 * k, 0.f);
    return;
  }
  // ---- one pass over the split's positions with an online softmax.  Lane
  // (g, cidx) handles position j = j0 + g of each pass and dims cidx*8..+7:
  // a 16-byte K chunk and a 16-byte V chunk per pass; the LPP lanes of a
  // position sum their partial dot products; every lane keeps a running
  // (max, sum, weighted V) for its positions, and the PPP groups are merged by
  // log-sum-exp at the end.  The new row takes part like a cached one (its
  // chunk is selected in registers), so the pass has no divergent branch.
  constexpr int LPP = HD / 8;
  constexpr int PPP = 64 / LPP;
  constexpr int U = HD == 128 ? 8 : 4;  // passes whose loads are issued together
  const int gi = lane / LPP, cidx = lane % LPP;
  float qc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qc[e] = qs[cidx * 8 + e];
  uint4 knq = make_uint4(0u, 0u, 0u, 0u), vnq = knq;
  if (has_new) {
    const u32x4 a4 = ((const LDS u32x4*)kn)[cidx], b4 = ((const LDS u32x4*)vn)[cidx];
    knq = make_uint4(a4.x, a4.y, a4.z, a4.w);
    vnq = make_uint4(b4.x, b4.y, b4.z, b4.w);
  }
  // head_dim 64: q as bf16 high and low parts, so that a K chunk's dot products
  // run on v_dot2 (bf16 pairs, exact products, fp32 accumulate) without
  // converting K (Llama-1B -7 us, batch 16 -17 us; the head_dim 128 build lost
  // 22 us on Qwen3-8B with it and keeps the fp32 FMAs)
  bf16x2 qhi[4], qlo[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h0 = (__bf16)qc[2 * e], h1 = (__bf16)qc[2 * e + 1];
    qhi[e] = bf16x2{h0, h1};
    qlo[e] = bf16x2{(__bf16)(qc[2 * e] - (float)h0), (__bf16)(qc[2 * e + 1] - (float)h1)};
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  for (int j0 = 0; j0 < n; j0 += U * PPP) {
    uint4 ku[U], vu[U];
    if (nk > 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        int j = j0 + u * PPP + gi;
        j = j < nk ? j : nk - 1;
        ku[u] = src.ld16(0, j * HD * 2 + cidx * 16);
        vu[u] = src.ld16(1, j * HD * 2 + cidx * 16);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) ku[u] = vu[u] = knq;
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch's LDS reads stay in flight together
    // the U scores first, then one rescale of the running sums per pass: the
    // exponentials of a pass do not wait on one another
    float sc[U];
    float mx = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * PPP + gi;
      // the new row (j == nk) or past the end (masked below): the new row's chunk
      const bool cached = j < nk;
      const uint4 k4 = make_uint4(cached ? ku[u].x : knq.x, cached ? ku[u].y : knq.y, cached ? ku[u].z : knq.z,
                                  cached ? ku[u].w : knq.w);
      float d = 0.f;
      if (HD == 64) {
        const bf16x2 k0 = __builtin_bit_cast(bf16x2, k4.x), k1 = __builtin_bit_cast(bf16x2, k4.y);
        const bf16x2 k2 = __builtin_bit_cast(bf16x2, k4.z), k3 = __builtin_bit_cast(bf16x2, k4.w);
        d = __builtin_amdgcn_fdot2_f32_bf16(k0, qhi[0], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k1, qhi[1], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k2, qhi[2], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k3, qhi[3], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k0, qlo[0], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k1, qlo[1], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k2, qlo[2], d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(k3, qlo[3], d, false);
      } else {
        d = fmaf(bf16lo(k4.x), qc[0], d); d = fmaf(bf16hi(k4.x), qc[1], d);
        d = fmaf(bf16lo(k4.y), qc[2], d); d = fmaf(bf16hi(k4.y), qc[3], d);
        d = fmaf(bf16lo(k4.z), qc[4], d); d = fmaf(bf16hi(k4.z), qc[5], d);
        d = fmaf(bf16lo(k4.w), qc[6], d); d = fmaf(bf16hi(k4.w), qc[7], d);
      }
      // sum over the LPP lanes of this position (8: half a DPP row, 16: a row)
      d += dppf<DppXor1>(d);
      d += dppf<DppXor2>(d);
      d += dppf<DppHalfMirror>(d);
      if (LPP == 16) d += dppf<DppRor8>(d);
      sc[u] = j < n ? d * c.inv_sqrt_hd : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
    // a finite base while no position of this lane group is valid yet (then
    // every term below is zero and the sums stay empty)
    const float mb = mx == -INFINITY ? 0.f : mx;
    const float al = __expf(m - mb);  // 0 when m = -inf
    l *= al;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= al;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * PPP + gi;
      const float pj = __expf(sc[u] - mb);  // 0 for masked positions
      const bool cached = j < nk;
      const uint4 v4 = make_uint4(cached ? vu[u].x : vnq.x, cached ? vu[u].y : vnq.y, cached ? vu[u].z : vnq.z,
                                  cached ? vu[u].w : vnq.w);
      const float vf[8] = {bf16lo(v4.x), bf16hi(v4.x), bf16lo(v4.y), bf16hi(v4.y),
                           bf16lo(v4.z), bf16hi(v4.z), bf16lo(v4.w), bf16hi(v4.w)};
      l += pj;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(pj, vf[e], o[e]);
    }
    m = mx;
  }
  // merge the PPP position groups: lane l with lane l ^ mm, by DPP within a
  // 16-lane row (mm = 8) and the gfx950 row/half swaps across rows (16, 32)
#pragma unroll
  for (int mm = LPP; mm < 64; mm <<= 1) {
    auto other = [&](float v) {
      if (mm == 8) return dppf<DppRor8>(v);
      if (mm == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        return __uint_as_float((lane & 16) ? r[0] : r[1]);
      }
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
      return __uint_as_float((lane & 32) ? r[0] : r[1]);
    };
    const float m2 = other(m);
    const float l2 = other(l);
    float o2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o2[e] = other(o[e]);
    const float M = fmaxf(m, m2);
    const float a1 = m == -INFINITY ? 0.f : __expf(m - M);
    const float a2 = m2 == -INFINITY ? 0.f : __expf(m2 - M);
    l = l * a1 + l2 * a2;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = o[e] * a1 + o2[e] * a2;
    m = M;
  }
  if (lane == 0) {
    st_agent(outp, m);
    st_agent(outp + 1, l);
  }
  if (gi == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) st_agent(outp + 2 + cidx * 8 + e, o[e]);
  }
  if (tr && lane == 0) tr[7] = now_ticks();
}

// Batched attention, head_dim 64, on the matrix cores: the four compute waves
// of the group take the split's chunks of 32 positions in turn (wave w chunks
// w, w + 4, ...), for every query head of the kv group at once:
//   scores  S = K q^T with v_mfma_f32_16x16x32_bf16 per 16 positions: A = the
//           K rows (lane l: position l % 16, dims 8 (l / 16) .. +7, one 16-byte
//           LDS read), B = q^T (lane l: head l % 16, the same dims; heads past
//           the group's are zero; q as bf16 high and low parts, two MFMAs), so
//           lane (head h = l % 16, g = l / 16) holds h's scores of positions
//           4 g .. 4 g + 3;
//   softmax online per head (running max and sum; the four lanes of a head
//           combine by row swaps);
//   P V     O += P V per 16 head dims: A = P (lane l: head l % 16, positions
//           8 (l / 16) .. +7: the score layout of two 16-position blocks
//           regrouped by one permlane32 and one permlane16 swap; P as bf16
//           high and low parts, two MFMAs), B = V (lane l: dim l % 16, the same
//           positions, two ds_read_b64_tr_b16 of the position-major V rows).
// The cached rows arrive in the interleaved tile layout (Tile::ilv: chunk j's
// K and V rows in ring page j / 2): a wave waits for its chunk's page, and
// after each round of four chunks every wave hands back that round's two pages
// (pages.wait(p), pages.release(p0, p1)), so the loaders refill the ring while
// the task runs.  The new K/V row (scratch of each wave) is read instead of
// the ring for its position, and so are the masked positions of a chunk that
// holds no cached row (any other masked position reads its chunk's first row:
// finite values whose weight is zero).  The waves then exchange their
// per-head (max, sum, O) through the instruction's partial-sum slot (xarea, 12
// x 66 floats: wave w's partials of heads h != w) and wave h merges head h's
// four and stores the split partial.  sync(k): the group's k-th rendezvous
// (all four waves past it).
template <int POL = 0, class Src, class Sync, class Pages>
__device__ inline void attn_mfma64(const Src& src, const Meta& mt, const Consts& c, int cw, LDS float* gscr,
                                   LDS float* xarea, bool writer, const Sync& sync, const Pages& pages,
                                   unsigned long long* tr = nullptr) {
  constexpr int HD = 64;
  const int lane = lane_id();
  LDS float* scr = gscr + cw * kScratch;
  const AttnTask at = attn_prologue<HD, POL>(mt, c, cw, scr, writer);
  const int nk = at.nk, hpg = c.hpg;
  const int n = nk + (at.has_new ? 1 : 0);
  const LDS uint16_t* kn = (const LDS uint16_t*)(scr + HD);
  const LDS uint16_t* vn = (const LDS uint16_t*)(scr + 2 * HD);
  sync(1);  // every wave's rotated q is in its scratch
  if (tr && lane == 0) tr[6] = now_ticks();
  const int hq = lane & 15, gq = lane >> 4;
  // B operands of the scores: q^T, head hq, dims 32 kb + 8 gq .. +7
  bf16x8 qh[2], ql[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = hq < hpg ? gscr[hq * kScratch + 32 * kb + 8 * gq + e] : 0.f;
      const __bf16 h = (__bf16)v;
      qh[kb][e] = h;
      ql[kb][e] = (__bf16)(v - (float)h);
    }
  }
  const int nch = (n + 31) >> 5;                      // chunks of the split
  const int npg = (((nk + 31) >> 5) + 1) >> 1;        // ring pages of its cached rows
  float m_run = -INFINITY, l_run = 0.f;  // head hq's, in lanes (hq, any gq)
  f32x4 O[4];                            // O[db]: lane l: dim 16 db + l % 16, heads 4 (l / 16) + j
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto other16 = [&](float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
  };
  auto other32 = [&](float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float((lane & 32) ? r[0] : r[1]);
  };
  // the new row's K chunks of this lane (loop-invariant)
  const u32x4 kw0 = *(const LDS u32x4*)(kn + 8 * gq), kw1 = *(const LDS u32x4*)(kn + 32 + 8 * gq);
  for (int rd = 0; 4 * rd < nch; ++rd) {
    const int s0 = 32 * (4 * rd + cw);
    if (s0 >= n) {
      pages.release(2 * rd, 2 * rd + 2 < npg ? 2 * rd + 2 : npg);
      continue;
    }
    if (s0 < nk && !pages.wait(s0 >> 6)) return;
    // the row a lane reads for position pp: its own while cached, else the
    // chunk's first row while that is cached, else the scratch row
    auto ring_row = [&](int pp) { return pp < nk || (s0 < nk && !(at.has_new && pp == nk)); };
    auto row_of = [&](int pp) { return pp < nk ? pp : s0; };
    f32x4 S[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      const int pp = s0 + 16 * bk + hq;  // A row: position
      const bool rr_ = ring_row(pp);
      const int pr = row_of(pp);
      S[bk] = f32x4{0.f, 0.f, 0.f, 0.f};
      // a 128-byte row never straddles a 4 KiB block or the ring's end
      const uint32_t krow = src.addr(0, (uint32_t)(pr * HD * 2)) + (uint32_t)(16 * gq);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 kr = *(const LDS u32x4*)(uintptr_t)(krow + 64 * kb);
        const u32x4 ka = rr_ ? kr : (kb ? kw1 : kw0);
        const bf16x8 a = __builtin_bit_cast(bf16x8, ka);
        S[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[kb], S[bk], 0, 0, 0);
        S[bk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[kb], S[bk], 0, 0, 0);
      }
    }
    // scores of lane (hq, gq): positions s0 + 16 bk + 4 gq + j
    float sc[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pp = s0 + 16 * bk + 4 * gq + j;
        sc[bk][j] = pp < n ? S[bk][j] * c.inv_sqrt_hd : -INFINITY;
        mx = fmaxf(mx, sc[bk][j]);
      }
    mx = fmaxf(mx, other16(mx));
    mx = fmaxf(mx, other32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __expf(m_run - base);  // 0 when m_run = -inf
    float P[2][4], rs = 0.f;
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        P[bk][j] = __expf(sc[bk][j] - base);  // 0 for masked positions
        rs += P[bk][j];
      }
    rs += other16(rs);
    rs += other32(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    // rescale O: row j of every block holds head 4 (l / 16) + j; head j's
    // factor sits in lane j (head j, group 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float aj = readlane_f(alpha, j);
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db][j] *= aj;
    }
    // regroup P into the A layout: lane (h, g) gets positions 8 g .. 8 g + 7
    float pa[4], pb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(P[0][j]), __float_as_uint(P[1][j]), false, false);
      const auto r16 = __builtin_amdgcn_permlane16_swap(r32[0], r32[1], false, false);
      pa[j] = __uint_as_float(r16[0]);
      pb[j] = __uint_as_float(r16[1]);
    }
    bf16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = e < 4 ? pa[e] : pb[e - 4];
      const __bf16 h = (__bf16)v;
      ph[e] = h;
      pl[e] = (__bf16)(v - (float)h);
    }
    // V: lane L = 16 g + 4 r + cc addresses row s0 + 8 g + 4 half + r, dims
    // 16 db + 4 cc .. +3; the transposed read hands lane (g, q) the 4 rows'
    // dim 16 db + q
    const int rg = lane >> 4, rr = (lane >> 2) & 3, cc = lane & 3;
    // each half's V row address once (a row never straddles a 4 KiB block or
    // the ring's end), the 16-dim blocks as offsets from it
    uint32_t vrow[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int pp = s0 + 8 * rg + 4 * half + rr;
      vrow[half] = ring_row(pp) ? src.addr(1, (uint32_t)(row_of(pp) * HD * 2)) : (uint32_t)(uintptr_t)vn;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      bf16x4 vh[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
        vh[half] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS bf16x4*)(uintptr_t)(vrow[half] + (16 * db + 4 * cc) * 2));
      bf16x8 vb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vb[e] = vh[0][e];
        vb[4 + e] = vh[1][e];
      }
      O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, O[db], 0, 0, 0);
      O[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, O[db], 0, 0, 0);
    }
    // this round's pages: every wave has read its chunk (release waits for the
    // LDS reads to return)
    pages.release(2 * rd, 2 * rd + 2 < npg ? 2 * rd + 2 : npg);
  }
  // exchange: wave w's (max, sum, O) of head h != w at slot w * 3 + (h < w ? h : h - 1)
  auto slot = [&](int w, int h) { return xarea + (w * 3 + (h < w ? h : h - 1)) * (HD + 2); };
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if (h >= hpg || h == cw) continue;
    LDS float* xs = slot(cw, h);
    const float mh = readlane_f(m_run, h), lh = readlane_f(l_run, h);
    if (lane == 0) {
      xs[0] = mh;
      xs[1] = lh;
    }
    if (lane < 16) {
#pragma unroll
      for (int db = 0; db < 4; ++db) xs[2 + 16 * db + lane] = O[db][h];
    }
  }
  sync(2);  // every wave's partials are in the slot
  if (cw >= hpg) return;
  // head cw: merge the four quarters (own registers + three slots), then store
  const float mo = readlane_f(m_run, cw), lo_ = readlane_f(l_run, cw);
  float mw[4], lw[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w == cw) {
      mw[w] = mo;
      lw[w] = lo_;
    } else {
      const LDS float* xs = slot(w, cw);
      mw[w] = xs[0];
      lw[w] = xs[1];
    }
  }
  const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
  float aw[4], L = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    aw[w] = (mw[w] == -INFINITY) ? 0.f : __expf(mw[w] - M);
    L += aw[w] * lw[w];
  }
  GLB float* outp = (GLB float*)mt.q(AttnOut) + ((((size_t)at.b * c.nkv + at.g) * c.S + at.s) * c.hpg + cw) * (HD + 2);
  if (lane == 0) {
    st_agent(outp, M);
    st_agent(outp + 1, L);
  }
  if (lane < 16) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float ow = (w == cw) ? O[db][cw] : slot(w, cw)[2 + 16 * db + lane];
        o += aw[w] * ow;
      }
      st_agent(outp + 2 + 16 * db + lane, o);
    }
  }
  if (tr && lane == 0) tr[7] = now_ticks();
}

// Merge the S split partials of one query head (log-sum-exp).  Lane s reads
// split s's (max, sum) and turns it into a weight; the weighted outputs are
// read 32 splits per batch with clamped (branch-free) addresses.  The first
// batch is issued right behind the (max, sum) loads, before the weights are
// formed, so up to 32 splits cost one memory round trip.
template <int HD, int POL = 0>
__device__ inline void combine_wave(const Meta& m, const Consts& c, int cw,
                                    unsigned long long* tr = nullptr) {
  if (cw >= c.hpg) return;
  const int lane = lane_id();
  const int b = m.w(WGx), g = m.w(WGy);
  constexpr int PER = HD / 64;
  constexpr int UB = 32;  // splits per batch of loads
  const GLB float* part = (const GLB float*)m.q(CombPart) + (((size_t)b * c.nkv + g) * c.S * c.hpg + cw) * (HD + 2);
  const size_t stride = (size_t)c.hpg * (HD + 2);
  const int S = c.S;  // <= 64 (checked at plan build)
  const int sl = lane < S ? lane : S - 1;
  const CohT<kCohPolicy> cp(part);  // blocks of different events share lines
  const float ms = cp.f1((uint32_t)(sl * stride) * 4), ls = cp.f1((uint32_t)(sl * stride + 1) * 4);
  float M = 0.f, wsp = 0.f, L = 0.f;
  float o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int s0 = 0; s0 < S; s0 += UB) {
    float ov[UB][PER];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int s = s0 + u < S ? s0 + u : S - 1;
#pragma unroll
      for (int k = 0; k < PER; ++k) ov[u][k] = cp.f1((uint32_t)(2 + lane + 64 * k) * 4, (uint32_t)(s * stride) * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (s0 == 0) {  // the (max, sum) loads were issued first: no wait for the batch
      const bool live = lane < S && ls > 0.f;
      M = wave_max(live ? ms : -INFINITY);
      wsp = live ? __expf(ms - M) : 0.f;
      L = wave_sum(wsp * (live ? ls : 0.f));
      if (tr && lane == 0) tr[6] = now_ticks();
    }
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const float w = readlane_f(wsp, s0 + u < 64 ? s0 + u : 63);  // 0 for splits >= S
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = fmaf(s0 + u < S ? w : 0.f, ov[u][k], o[k]);
    }
  }
  GLB float* out = (GLB float*)m.q(CombOut);
  const int k0 = (g * c.hpg + cw) * HD;
  if (c.B == 1) {
#pragma unroll
    for (int k = 0; k < PER; ++k) st_agent(out + k0 + lane + 64 * k, o[k] / L);
    return;
  }
  // batch > 1: split for the O projection's tiles; lane ch < HD / 8 gathers
  // chunk ch (elements 8 ch .. 8 ch + 7, held by lanes 8 ch % 64 + e of o[8 ch / 64])
  float v[8];
  const int ch = lane < HD / 8 ? lane : 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const float s2 = __shfl(o[k], (8 * ch) % 64 + e, 64);
      if ((8 * ch) / 64 == k) t = s2;
    }
    v[e] = t / L;
  }
  if (lane < HD / 8) {
    u32x4 hi, lo;
    split8(v, hi, lo);
    const uint32_t so = split_off(b, k0 + 8 * ch, c.B);
    st_agent16((const GLB void*)out, so, __builtin_bit_cast(f32x4, hi));
    st_agent16((const GLB void*)out, so + 16, __builtin_bit_cast(f32x4, lo));
  }
}

// Reduce the LM-head tile maxima of sequence b in tile order, lowest index on
// ties.  Compute wave cw scans the contiguous quarter cw of the T tile maxima,
// 32 per lane per batch (every load of a batch issued before any is used), and
// leaves its best (value, index) in out2[0..1]; argmax_final merges the quarters.
template <int POL = 0>
__device__ inline void argmax_part(const Meta& m, const Consts& c, int cw, LDS float* out2) {
  const int lane = lane_id();
  const int b = m.w(WGx), T = m.w(WPay);
  const CohT<POL> mx((const GLB f32x2*)m.q(AmMax) + (size_t)b * T);
  const int per = (T + kNW - 1) / kNW;
  const int lo = cw * per, hi = lo + per < T ? lo + per : T;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  constexpr int U = 32;
  for (int t0 = lo; t0 < hi; t0 += 64 * U) {
    f32x2 pr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * 64 + lane;
      pr[u] = mx.f2((uint32_t)(t < hi ? t : lo) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * 64 + lane;
      const int i = __float_as_int(pr[u].y);
      if (t < hi && amax_better(pr[u].x, i, bv, bi)) {
        bv = pr[u].x;
        bi = i;
      }
    }
  }
#pragma unroll
  for (int msk = 32; msk >= 1; msk >>= 1) {
    const float ov = __shfl_xor(bv, msk, 64);
    const int oi = __shfl_xor(bi, msk, 64);
    if (amax_better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    out2[0] = bv;
    out2[1] = __int_as_float(bi);
  }
}
// part[w * stride + 0..1]: wave w's (value, index); one wave stores the winner.
__device__ inline void argmax_final(const Meta& m, const LDS float* part, int stride) {
  float bv = part[0];
  int bi = __float_as_int(part[1]);
#pragma unroll
  for (int w = 1; w < kNW; ++w) {
    const float v = part[w * stride];
    const int i = __float_as_int(part[w * stride + 1]);
    if (amax_better(v, i, bv, bi)) {
      bv = v;
      bi = i;
    }
  }
  if (lane_id() == 0) ((GLB int*)m.q(AmOut))[m.w(WGx)] = bi;
}

}  // namespace mkd
