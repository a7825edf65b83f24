// Device-side definitions shared by the persistent interpreter and the
// layerwise kernels: constants, instruction decoding, tile byte layout and the
// tile arithmetic of every operator of the Llama-family decode step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mkd {

// ---- instruction words (same layout as the host planner) -------------------
enum : int {
  WOpcode = 0, WSpec = 1, WOpRow = 2, WWaitCnt = 3, WWaitEv = 4, WWaitTgt = 5, WSigCnt = 6, WSigEv = 7,
  WSigInc = 8, WTask = 9, WLayer = 10, WGx = 11, WGy = 12, WGz = 13, WPay = 14
};
enum : int { OpNoop = 0, OpQkv = 1, OpAttn = 2, OpCombine = 3, OpOproj = 4, OpGateUp = 5, OpDown = 6, OpLmHead = 7, OpArgmax = 8 };

// ---- operand table slots (one row of 16 u64 per op) --------------------------
enum : int {
  // QKV
  QkvWq = 0, QkvWk = 1, QkvWv = 2, QkvNorm = 3, QkvX = 4, QkvEmbed = 5, QkvTokens = 6, QkvOut = 7,
  // ATTN
  AttnQkv = 0, AttnK = 1, AttnV = 2, AttnRope = 3, AttnOut = 4, AttnQn = 5, AttnKn = 6,
  // COMBINE
  CombPart = 0, CombOut = 1,
  // OPROJ
  OWo = 0, OIn = 1, OX = 2, OEmbed = 3, OTokens = 4, OOut = 5,
  // GATEUP
  GuWg = 0, GuWu = 1, GuNorm = 2, GuIn = 3, GuOut = 4,
  // DOWN
  DnW = 0, DnIn = 1, DnRes = 2, DnOut = 3,
  // LMHEAD
  LmW = 0, LmNorm = 1, LmIn = 2, LmLogits = 3, LmMax = 4,
  // ARGMAX
  AmMax = 0, AmOut = 1
};

constexpr int kPage = 16384;  // bytes per LDS page
constexpr int kNumPages = 9;  // page ring of the interpreter: 144 KiB
constexpr int kNW = 4;        // compute waves per workgroup (K split / one q head each)
constexpr int kMaxRows = 16;  // weight rows per GEMV tile
constexpr int kMaxChunks = 6; // 16-byte activation chunks per lane (K / (8 * kNW * 64))
constexpr int kScratch = 512; // floats of per-compute-wave scratch

struct Consts {
  int H, nq, nkv, hd, F, V, L, B, cap, hpg, RPG, S, T_v, qk_norm;
  float eps, inv_sqrt_hd;
};

struct KArgs {
  const int* queue;           // [C][max_len][32]
  const uint64_t* optab;      // [num_ops][16]
  unsigned* counters;         // [num_events]
  unsigned* err;              // watchdog record [8]
  unsigned long long* trace;  // [C][max_len][4] or null
  int max_len;
  unsigned epoch;
  unsigned long long timeout_ticks;
  Consts c;
};

// ---- small helpers -----------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// token id of sequence 0, clamped into [0, vocab) so that a bad id cannot index
// outside the embedding
__device__ __forceinline__ int token0(const uint64_t tokens_ptr, int V) {
  int t = ((const int*)tokens_ptr)[0];
  return t < 0 ? 0 : (t >= V ? V - 1 : t);
}
__device__ __forceinline__ int ld_word(const int* ins, int w) { return ins[w]; }
__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ---- tile byte layout ---------------------------------------------------------
// A tile's weight bytes are one or two contiguous source segments placed one
// after the other in the tile's buffer, the second at a 1 KiB boundary.  Plain
// scalars (no arrays) so that nothing is indexed at run time and everything
// stays in registers.
struct Tile {
  const char* p0;
  const char* p1;
  int len0, off1, len1;
  int bytes, npages;
};

__device__ __forceinline__ int round1k(int v) { return (v + 1023) & ~1023; }

__device__ inline Tile tile_info(const int* ins, const uint64_t* orow, const Consts& c) {
  Tile t;
  t.p0 = nullptr;
  t.p1 = nullptr;
  t.len0 = t.off1 = t.len1 = 0;
  const int op = ins[WOpcode];
  switch (op) {
    case OpQkv: {
      const int g = ins[WGx], row0 = ins[WPay], nrows = ins[WPay + 1];
      const int qrows = c.hpg * c.hd;
      if (row0 < qrows)
        t.p0 = (const char*)orow[QkvWq] + ((size_t)g * qrows + row0) * c.H * 2;
      else if (row0 < qrows + c.hd)
        t.p0 = (const char*)orow[QkvWk] + ((size_t)g * c.hd + row0 - qrows) * c.H * 2;
      else
        t.p0 = (const char*)orow[QkvWv] + ((size_t)g * c.hd + row0 - qrows - c.hd) * c.H * 2;
      t.len0 = nrows * c.H * 2;
      break;
    }
    case OpOproj:
      t.p0 = (const char*)orow[OWo] + (size_t)ins[WPay] * c.nq * c.hd * 2;
      t.len0 = ins[WPay + 1] * c.nq * c.hd * 2;
      break;
    case OpGateUp:
      t.p0 = (const char*)orow[GuWg] + (size_t)ins[WPay] * c.H * 2;
      t.p1 = (const char*)orow[GuWu] + (size_t)ins[WPay] * c.H * 2;
      t.len0 = t.len1 = ins[WPay + 1] * c.H * 2;
      break;
    case OpDown:
      t.p0 = (const char*)orow[DnW] + (size_t)ins[WPay] * c.F * 2;
      t.len0 = ins[WPay + 1] * c.F * 2;
      break;
    case OpLmHead:
      t.p0 = (const char*)orow[LmW] + (size_t)ins[WPay] * c.H * 2;
      t.len0 = ins[WPay + 1] * c.H * 2;
      break;
    case OpAttn: {
      const int b = ins[WGx], g = ins[WGy], lo = ins[WPay], hi = ins[WPay + 1], pos = ins[WPay + 2];
      int nk = (hi < pos ? hi : pos) - lo;
      if (nk < 0) nk = 0;
      const size_t base = (((size_t)b * c.nkv + g) * c.cap + lo) * c.hd * 2;
      t.p0 = (const char*)orow[AttnK] + base;
      t.p1 = (const char*)orow[AttnV] + base;
      t.len0 = t.len1 = nk * c.hd * 2;
      break;
    }
    default:
      break;
  }
  t.off1 = round1k(t.len0);
  t.bytes = t.len1 ? t.off1 + t.len1 : t.len0;
  t.npages = (t.bytes + kPage - 1) / kPage;
  return t;
}

// ---- weight sources -------------------------------------------------------------
// LDS page ring: page j of the tile lives in ring slot (first + j) mod kNumPages.
struct LdsSrc {
  const char* ring;
  int first_slot;
  int off1;
  __device__ __forceinline__ const char* at(int seg, int o) const {
    const int t = (seg ? off1 : 0) + o;
    int slot = first_slot + (t >> 14);
    if (slot >= kNumPages) slot -= kNumPages;
    return ring + slot * kPage + (t & (kPage - 1));
  }
  __device__ __forceinline__ uint4 ld16(int seg, int o) const { return *(const uint4*)at(seg, o); }
  __device__ __forceinline__ uint16_t ld2(int seg, int o) const { return *(const uint16_t*)at(seg, o); }
};
// Straight from device memory (layerwise kernels).
struct GlbSrc {
  const char* p0;
  const char* p1;
  __device__ __forceinline__ uint4 ld16(int seg, int o) const { return *(const uint4*)((seg ? p1 : p0) + o); }
  __device__ __forceinline__ uint16_t ld2(int seg, int o) const { return *(const uint16_t*)((seg ? p1 : p0) + o); }
};

// ---- activations of a GEMV tile ---------------------------------------------
// Each compute wave owns about K / kNW consecutive input elements; lane l holds the
// 16-byte chunks l, l + 64, ... of that range as fp32 (times the RMSNorm
// weight when the op fuses a norm), plus its partial sum of squares.
struct Act {
  float x[kMaxChunks][8];
  float ss;
  int nc;
};

// src: fp32 vector (xf) or a bf16 row (xb); nw: bf16 norm weight or null
__device__ inline void load_act(Act& a, int K, int cw, const float* xf, const uint16_t* xb, const uint16_t* nw) {
  const int lane = lane_id();
  const int nch = K / 8;                    // 16-byte chunks of bf16 weights per row
  const int cpw = (nch + kNW - 1) / kNW;    // chunks per wave (the last wave may get fewer)
  const int base = cw * cpw;
  a.nc = (cpw + 63) / 64;
  a.ss = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int ch = lane + 64 * j;
#pragma unroll
    for (int e = 0; e < 8; ++e) a.x[j][e] = 0.f;
    if (j < a.nc && ch < cpw && base + ch < nch) {
      const int k0 = (base + ch) * 8;
      float v[8];
      if (xf) {
        float4 u0 = *(const float4*)(xf + k0), u1 = *(const float4*)(xf + k0 + 4);
        v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w; v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
      } else {
        uint4 u = *(const uint4*)(xb + k0);
        v[0] = bf16lo(u.x); v[1] = bf16hi(u.x); v[2] = bf16lo(u.y); v[3] = bf16hi(u.y);
        v[4] = bf16lo(u.z); v[5] = bf16hi(u.z); v[6] = bf16lo(u.w); v[7] = bf16hi(u.w);
      }
      float w[8];
      if (nw) {
        uint4 u = *(const uint4*)(nw + k0);
        w[0] = bf16lo(u.x); w[1] = bf16hi(u.x); w[2] = bf16lo(u.y); w[3] = bf16hi(u.y);
        w[4] = bf16lo(u.z); w[5] = bf16hi(u.z); w[6] = bf16lo(u.w); w[7] = bf16hi(u.w);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = 1.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a.ss += v[e] * v[e];
        a.x[j][e] = v[e] * w[e];
      }
    }
  }
}

// Partial dot products of the wave's K range for 'nrows' rows of a tile; rows
// r < n0 come from segment 0, the rest from segment 1 (row r - n0).  Row r's
// partial lands in part[r] (lane 0 writes).
template <class Src>
__device__ inline void gemv_rows(const Src& src, const Act& a, int K, int cw, int n0, int nrows, float* part) {
  const int lane = lane_id();
  const int nch = K / 8;
  const int cpw = (nch + kNW - 1) / kNW;
  const int base = cw * cpw;
  float acc[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int ch = lane + 64 * j;
    if (j < a.nc && ch < cpw && base + ch < nch) {
      const int cb = (base + ch) * 16;
#pragma unroll
      for (int r = 0; r < kMaxRows; ++r) {
        if (r < nrows) {
          const int seg = r < n0 ? 0 : 1;
          const int rr = r < n0 ? r : r - n0;
          uint4 u = src.ld16(seg, rr * K * 2 + cb);
          float s = acc[r];
          s = fmaf(bf16lo(u.x), a.x[j][0], s);
          s = fmaf(bf16hi(u.x), a.x[j][1], s);
          s = fmaf(bf16lo(u.y), a.x[j][2], s);
          s = fmaf(bf16hi(u.y), a.x[j][3], s);
          s = fmaf(bf16lo(u.z), a.x[j][4], s);
          s = fmaf(bf16hi(u.z), a.x[j][5], s);
          s = fmaf(bf16lo(u.w), a.x[j][6], s);
          s = fmaf(bf16hi(u.w), a.x[j][7], s);
          acc[r] = s;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r) {
    if (r < nrows) {
      float v = wave_sum(acc[r]);
      if (lane == 0) part[r] = v;
    }
  }
}

// Which activation and norm a GEMV op reads, and its K.
struct GemvIn {
  const float* xf;
  const uint16_t* xb;
  const uint16_t* nw;
  int K;
  int n0, nrows;  // rows in segment 0, total rows
};

__device__ inline GemvIn gemv_input(const int* ins, const uint64_t* orow, const Consts& c) {
  GemvIn g;
  g.xf = nullptr;
  g.xb = nullptr;
  g.nw = nullptr;
  const int op = ins[WOpcode];
  switch (op) {
    case OpQkv:
      g.K = c.H;
      g.nw = (const uint16_t*)orow[QkvNorm];
      if (orow[QkvX]) g.xf = (const float*)orow[QkvX];
      else g.xb = (const uint16_t*)orow[QkvEmbed] + (size_t)token0(orow[QkvTokens], c.V) * c.H;
      g.n0 = g.nrows = ins[WPay + 1];
      break;
    case OpOproj:
      g.K = c.nq * c.hd;
      g.xf = (const float*)orow[OIn];
      g.n0 = g.nrows = ins[WPay + 1];
      break;
    case OpGateUp:
      g.K = c.H;
      g.nw = (const uint16_t*)orow[GuNorm];
      g.xf = (const float*)orow[GuIn];
      g.n0 = ins[WPay + 1];
      g.nrows = 2 * ins[WPay + 1];
      break;
    case OpDown:
      g.K = c.F;
      g.xf = (const float*)orow[DnIn];
      g.n0 = g.nrows = ins[WPay + 1];
      break;
    default:  // OpLmHead
      g.K = c.H;
      g.nw = (const uint16_t*)orow[LmNorm];
      g.xf = (const float*)orow[LmIn];
      g.n0 = g.nrows = ins[WPay + 1];
      break;
  }
  return g;
}

// Epilogue of a GEMV tile, run by one wave once every compute wave's partials
// (part[w][r]) and partial sums of squares (ssp[w]) are in LDS.
__device__ inline void gemv_epilogue(const int* ins, const uint64_t* orow, const Consts& c, const float (*part)[kMaxRows],
                                     const float* ssp) {
  const int lane = lane_id();
  const int op = ins[WOpcode];
  const GemvIn g = gemv_input(ins, orow, c);
  float scale = 1.f;
  if (g.nw) {
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
  const int row0 = ins[WPay], nr = ins[WPay + 1];
  switch (op) {
    case OpQkv:
      if (lane < nr) ((float*)orow[QkvOut])[(size_t)ins[WGx] * c.RPG + row0 + lane] = v;
      break;
    case OpOproj:
      if (lane < nr) {
        float res = orow[OX] ? ((const float*)orow[OX])[row0 + lane]
                             : bf16f(((const uint16_t*)orow[OEmbed])[(size_t)token0(orow[OTokens], c.V) * c.H + row0 + lane]);
        ((float*)orow[OOut])[row0 + lane] = res + v;
      }
      break;
    case OpGateUp: {
      float u = __shfl(v, lane + nr, 64);  // up row j sits at tile row nr + j
      if (lane < nr) ((float*)orow[GuOut])[row0 + lane] = v / (1.f + __expf(-v)) * u;
      break;
    }
    case OpDown:
      if (lane < nr) ((float*)orow[DnOut])[row0 + lane] = ((const float*)orow[DnRes])[row0 + lane] + v;
      break;
    case OpLmHead: {
      if (lane < nr) ((float*)orow[LmLogits])[row0 + lane] = v;
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
        float* mx = (float*)orow[LmMax] + 2 * (size_t)ins[WGx];
        mx[0] = bv;
        ((int*)mx)[1] = bi;
      }
      break;
    }
    default:
      break;
  }
}

// ---- attention -----------------------------------------------------------------
// One wave per query head of the kv group: RoPE (and Qwen3's q/k RMSNorm), the
// new K/V row (written to the cache by wave 0 of the split that holds it),
// scores over the split's positions, and the partial (max, sum, weighted V).
template <int HD, class Src>
__device__ inline void attn_wave(const Src& src, const int* ins, const uint64_t* orow, const Consts& c, int cw,
                                 float* scr, bool writer) {
  const int lane = lane_id();
  const int b = ins[WGx], g = ins[WGy], s = ins[WGz];
  const int lo = ins[WPay], hi = ins[WPay + 1], pos = ins[WPay + 2];
  int nk = (hi < pos ? hi : pos) - lo;
  if (nk < 0) nk = 0;
  const bool has_new = pos >= lo && pos < hi;
  const float* qkv = (const float*)orow[AttnQkv] + ((size_t)b * c.nkv + g) * c.RPG;
  const float* rope = (const float*)orow[AttnRope] + (size_t)b * HD;  // (cos, sin) pairs
  float* qs = scr;            // rotated q, HD floats
  float* kn = scr + HD;       // new k (bf16-rounded), HD
  float* vn = scr + 2 * HD;   // new v (bf16-rounded), HD
  float* sc = scr + 3 * HD;   // scores
  constexpr int HALF = HD / 2;
  constexpr int PER = HD / 64;  // values per lane for a full head vector

  // rotate-half RoPE of head vector src (fp32, optional per-head RMSNorm with weight nw)
  auto rot = [&](const float* hv, const uint16_t* nw, float* out, bool round_bf16) {
    float v[PER];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      v[k] = hv[lane + 64 * k];
      ss += v[k] * v[k];
    }
    if (nw) {
      ss = wave_sum(ss);
      float inv = 1.f / sqrtf(ss / (float)HD + c.eps);
#pragma unroll
      for (int k = 0; k < PER; ++k) v[k] = v[k] * inv * bf16f(nw[lane + 64 * k]);
    }
    // stage in out[], then rotate pairs (i, i + HALF)
#pragma unroll
    for (int k = 0; k < PER; ++k) out[lane + 64 * k] = v[k];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    float r[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane + 64 * k;
      const int i = d < HALF ? d : d - HALF;
      const float cs = rope[2 * i], sn = rope[2 * i + 1];
      const float a = out[i], bb = out[i + HALF];
      r[k] = d < HALF ? a * cs - bb * sn : bb * cs + a * sn;
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int k = 0; k < PER; ++k) out[lane + 64 * k] = round_bf16 ? bf16f(f2bf(r[k])) : r[k];
    __builtin_amdgcn_wave_barrier();
  };

  const bool active = cw < c.hpg;
  if (active) {
    rot(qkv + cw * HD, c.qk_norm ? (const uint16_t*)orow[AttnQn] : nullptr, qs, false);
  }
  if (has_new) {
    // every wave computes the new row (cheap); the writer stores it
    rot(qkv + c.hpg * HD, c.qk_norm ? (const uint16_t*)orow[AttnKn] : nullptr, kn, true);
#pragma unroll
    for (int k = 0; k < PER; ++k) vn[lane + 64 * k] = bf16f(f2bf(qkv[(c.hpg + 1) * HD + lane + 64 * k]));
    __builtin_amdgcn_wave_barrier();
    if (writer) {
      size_t row = (((size_t)b * c.nkv + g) * c.cap + pos) * HD;
      uint16_t* K = (uint16_t*)orow[AttnK] + row;
      uint16_t* Vv = (uint16_t*)orow[AttnV] + row;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        K[lane + 64 * k] = f2bf(kn[lane + 64 * k]);
        Vv[lane + 64 * k] = f2bf(vn[lane + 64 * k]);
      }
    }
  }
  if (!active) return;
  const int n = nk + (has_new ? 1 : 0);
  float* outp = (float*)orow[AttnOut] + ((((size_t)b * c.nkv + g) * c.S + s) * c.hpg + cw) * (HD + 2);
  if (n == 0) {
    if (lane == 0) {
      outp[0] = -INFINITY;
      outp[1] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) outp[2 + lane + 64 * k] = 0.f;
    return;
  }
  // scores: LPP lanes per position, 8 dims (16 bytes) per lane
  constexpr int LPP = HD / 8;
  constexpr int PPP = 64 / LPP;
  const int p_in = lane / LPP, cidx = lane % LPP;
  float qv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] = qs[cidx * 8 + e];
  for (int j0 = 0; j0 < n; j0 += PPP) {
    const int j = j0 + p_in;
    float d = 0.f;
    if (j < nk) {
      uint4 u = src.ld16(0, j * HD * 2 + cidx * 16);
      d = bf16lo(u.x) * qv[0] + bf16hi(u.x) * qv[1] + bf16lo(u.y) * qv[2] + bf16hi(u.y) * qv[3] +
          bf16lo(u.z) * qv[4] + bf16hi(u.z) * qv[5] + bf16lo(u.w) * qv[6] + bf16hi(u.w) * qv[7];
    } else if (j < n) {
#pragma unroll
      for (int e = 0; e < 8; ++e) d += kn[cidx * 8 + e] * qv[e];
    }
#pragma unroll
    for (int m = LPP / 2; m >= 1; m >>= 1) d += __shfl_xor(d, m, 64);
    if (cidx == 0 && j < n) sc[j] = d * c.inv_sqrt_hd;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  float m = -INFINITY;
  for (int j = lane; j < n; j += 64) m = fmaxf(m, sc[j]);
  m = wave_max(m);
  float l = 0.f, o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int j = 0; j < n; ++j) {
    const float p = __expf(sc[j] - m);
    l += p;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int dd = lane + 64 * k;
      const float vv = j < nk ? bf16f(src.ld2(1, (j * HD + dd) * 2)) : vn[dd];
      o[k] = fmaf(p, vv, o[k]);
    }
  }
  if (lane == 0) {
    outp[0] = m;
    outp[1] = l;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) outp[2 + lane + 64 * k] = o[k];
}

// Merge the S split partials of one query head (log-sum-exp).
template <int HD>
__device__ inline void combine_wave(const int* ins, const uint64_t* orow, const Consts& c, int cw) {
  if (cw >= c.hpg) return;
  const int lane = lane_id();
  const int b = ins[WGx], g = ins[WGy];
  constexpr int PER = HD / 64;
  const float* part = (const float*)orow[CombPart] + (((size_t)b * c.nkv + g) * c.S * c.hpg + cw) * (HD + 2);
  const size_t stride = (size_t)c.hpg * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < c.S; ++s) {
    const float* p = part + s * stride;
    if (p[1] > 0.f) M = fmaxf(M, p[0]);
  }
  float L = 0.f, o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.f;
  for (int s = 0; s < c.S; ++s) {
    const float* p = part + s * stride;
    if (!(p[1] > 0.f)) continue;
    const float w = __expf(p[0] - M);
    L += w * p[1];
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] = fmaf(w, p[2 + lane + 64 * k], o[k]);
  }
  float* out = (float*)orow[CombOut] + (size_t)b * c.nq * HD + (size_t)(g * c.hpg + cw) * HD;
#pragma unroll
  for (int k = 0; k < PER; ++k) out[lane + 64 * k] = o[k] / L;
}

// Reduce the LM-head tile maxima of sequence b in tile order (lowest index on ties).
__device__ inline void argmax_wave(const int* ins, const uint64_t* orow, const Consts& c) {
  const int lane = lane_id();
  const int b = ins[WGx], T = ins[WPay];
  const float* mx = (const float*)orow[AmMax] + (size_t)b * 2 * T;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int t = lane; t < T; t += 64) {
    float v = mx[2 * t];
    int i = ((const int*)mx)[2 * t + 1];
    if (v > bv || (v == bv && i < bi)) {
      bv = v;
      bi = i;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(bv, m, 64);
    int oi = __shfl_xor(bi, m, 64);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) ((int*)orow[AmOut])[b] = bi;
}

}  // namespace mkd
