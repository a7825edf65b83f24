// Tile arithmetic of the GLM-style pre-attention path (fp8 weights, M <= 16
// token rows): the operators of the MegaRTP article (tahou.com), sections 1
// and 4 -- fused add + RMSNorm + fp8 quant one token row per tile (A0), fp8
// GEMM tiles cut along the output rows (QKV-A, head gate and indexer-K hang
// off A0 independently; QKV-B and indexer-Q off the q path's norm + requant),
// RoPE on the last rope dims of each query head and the KV / indexer cache
// write-back.
//
// Formats: weights are OCP FP8 E4M3 codes [N, K] with an fp32 scale per 128 x 128
// block; activations are E4M3 codes with an fp32 scale per (token row, 128
// columns): s = max(amax, 1e-4) / 448.  A GEMM tile is 16 weight rows x M
// tokens on the matrix cores, one v_mfma_scale_f32_16x16x128_f8f6f4 per
// 128-column block (unit block scales: the product of the two fp8 operands is
// exact), the fp32 block result scaled by weight scale x token scale and
// accumulated.  Each compute wave owns a quarter of the 128-column blocks; the
// storer sums the four partial 16 x 16 blocks in fixed order.
#pragma once
#include "mk_device.hpp"

namespace mkd {

typedef int v8i __attribute__((ext_vector_type(8)));

// a GEMM tile: 16 weight rows, partials of the four compute waves summed by the
// storer (the head gate's K-split tiles included; its reduce op is a row op)
__device__ __forceinline__ bool glm_is_gemm(int op) {
  return op == OpGQkva || op == OpGGate || op == OpGIdxk || op == OpGQkvb || op == OpGIdxq;
}

// fp32 -> E4M3 code, round to nearest even, saturating at +-448 (largest
// finite E4M3).  Normal results round the fp32 significand at bit 20 (3
// fraction bits kept), a carry moving into the exponent; below 2^-6 the
// result is a multiple of 2^-9 (subnormal codes 0..8, 8 being the smallest
// normal).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.f);
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.f);
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  const uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}
// E4M3 code -> bf16 bits (exact: at most 4 significant bits; no NaN codes in weights)
__device__ __forceinline__ uint32_t e4m3_to_bf16(uint32_t c) {
  const uint32_t s = (c & 0x80u) << 8, e = (c >> 3) & 15u, m = c & 7u;
  if (e) return s | ((e + 120u) << 7) | (m << 4);
  return s | (__float_as_uint((float)m * 0.001953125f) >> 16);
}

// ---- fp8 GEMM tile, one compute wave's quarter of K --------------------------
// Lane l: weight row (tile row) l % 16 and token l % 16 for the operands; the
// lanes l / 16 = g hold bytes g*32 .. g*32+31 of each 128-column block for both
// operands (the same K positions, so the product sums over the whole block).
// Rows past the tile re-read its last row and tokens past M re-read token 0;
// those outputs are never stored.  Partial block: part[(4 g + i) * 16 + b].
template <int POL = 0, class Src>
__device__ inline void glm_gemm_wave(const Src& src, const Meta& m, const Consts& c, int cw, LDS float* part,
                                     unsigned long long* tr = nullptr) {
  const int op = m.w(WOpcode);
  const int lane = lane_id();
  const int K = (op == OpGQkvb || op == OpGIdxq) ? c.ql : c.H;
  const int nkb = K / 128, per = (nkb + kNW - 1) / kNW;
  const int kb0 = cw * per, kb1 = kb0 + per < nkb ? kb0 + per : nkb;
  const int row0 = m.w(WPay), nrows = m.w(WPay + 1);
  const int trows = m.w(WPay + 2) >= 0 ? 2 * nrows : nrows;
  const int r = lane & 15, g = lane >> 4, b = lane & 15;
  const int rc = r < trows ? r : trows - 1;
  const int seg = rc < nrows ? 0 : 1, rr = rc < nrows ? rc : rc - nrows;
  const int bb = b < c.B ? b : 0;
  // every row of a tile lies in one 128-row scale block (tiles of 16 rows at
  // multiples of 16; a RoPE-pair tile spans the rope dims of one head, which
  // never cross a multiple of 128 for head_dim 192 / rope 64 -- checked on the host)
  const GLB float* ws = (const GLB float*)m.q(GmS) + (size_t)(row0 / 128) * nkb;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (op == OpGGate) {
    // a K-split tile: blocks [gkb0, gkb0 + gnkb), one per compute wave; its rows
    // sit gnkb * 128 bytes apart in the LDS tile (in memory: K bytes apart).
    // The gate reads the unquantized fp32 norm output: bf16 high and low parts
    // against the exactly converted weights, 4 k-steps of 8 per lane per block.
    // The k order within a block is permuted (the same way for both operands,
    // so the block's sum is unchanged): load t of lane (token, g) takes the 4
    // activations at 16 t + 4 g, so the four g lanes of a token read 64
    // contiguous bytes; k-step ks uses loads 2 ks and 2 ks + 1, and the weight
    // bytes at the same positions.
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const CohT<POL> cx((const GLB float*)m.q(GmAF));
    const uint32_t xo = (uint32_t)(bb * K) * 4;
    const int gkb0 = m.w(WPay + 3), gnkb = m.w(WPay + 4);
    const int lrow = Src::kLds ? gnkb * 128 : K;  // bytes between the tile's rows in src
    constexpr int UG = 1;  // blocks whose weight and activation loads are issued together
    for (int kq = gkb0 + cw; kq < gkb0 + gnkb; kq += kNW * UG) {
      uint32_t wd[UG][8];
      f32x4 xa[UG][8];
      float sc[UG];
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        const int kb = kq + u * kNW < gkb0 + gnkb ? kq + u * kNW : kq;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int kl = 16 * t + 4 * g;
          wd[u][t] = src.ld4(seg, rr * lrow + (kb - gkb0) * 128 + kl);
          xa[u][t] = cx.f4(xo + (uint32_t)(kb * 128 + kl) * 4);
        }
        sc[u] = kq + u * kNW < gkb0 + gnkb ? ws[kb] : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);  // one memory latency per group of blocks
      if (tr && kq == gkb0 + cw && lane == 0) {
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        tr[6] = now_ticks();
      }
#pragma unroll
      for (int u = 0; u < UG; ++u) {
        f32x4 blk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f32x4 x0 = xa[u][2 * ks], x1 = xa[u][2 * ks + 1];
          const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          bf16x8 av, hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t code = (wd[u][2 * ks + e / 4] >> (8 * (e & 3))) & 0xFFu;
            av[e] = __builtin_bit_cast(__bf16, (uint16_t)e4m3_to_bf16(code));
            const __bf16 h = (__bf16)v[e];
            hi[e] = h;
            lo[e] = (__bf16)(v[e] - (float)h);
          }
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hi, blk, 0, 0, 0);
          blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, lo, blk, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(blk[i], sc[u], acc[i]);
      }
    }
  } else {
    const CohT<POL> ca((const GLB uint8_t*)m.q(GmA8)), cs((const GLB float*)m.q(GmAS));
    const uint32_t ao = (uint32_t)(bb * K), so = (uint32_t)(bb * nkb) * 4;
    constexpr int U = 4;  // blocks whose loads are issued together
    for (int kq = kb0; kq < kb1; kq += U) {
      v8i A[U], X[U];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kb = kq + u < kb1 ? kq + u : kb0;
        const int ko = kb * 128 + g * 32;
        const uint4 w0 = src.ld16(seg, rr * K + ko), w1 = src.ld16(seg, rr * K + ko + 16);
        const u32x4 x0 = ca.u4(ao + ko), x1 = ca.u4(ao + ko + 16);
        A[u] = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        X[u] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        sc[u] = kq + u < kb1 ? ws[kb] * cs.f1(so + kb * 4) : 0.f;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        // format codes 0 / 0: both operands E4M3; block scales 127 = 2^0
        const f32x4 blk = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[u], X[u], z, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(blk[i], sc[u], acc[i]);
      }
    }
  }
  if (tr && lane == 0) tr[7] = now_ticks();
#pragma unroll
  for (int i = 0; i < 4; ++i) part[(4 * g + i) * kMB + b] = acc[i];
}

// Quantize one 8-element chunk (lane) of a 128-element block held by 16
// consecutive lanes.  u is the row before its 1/rms factor inv (n = u * inv):
// the block's scale is max(max|n|, 1e-4) / 448 and each code is E4M3 of n / s,
// taken as 448 u / max|u| (the factor cancels) with a correctly rounded
// division, so that when that quotient is exactly representable -- as exact
// e4m3 ties of bf16-derived rows are -- the code is decided on the exact value.
// Returns the eight codes packed little-endian; *scale gets the block's scale.
__device__ __forceinline__ uint2 glm_quant8(const float (&u)[8], float inv, float* scale) {
  float amu = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amu = fmaxf(amu, fabsf(u[e]));
  amu = row_max16(amu);
  const float amn = amu * inv;
  const bool floor = !(amn >= 1e-4f);
  *scale = (floor ? 1e-4f : amn) / 448.f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = floor ? u[e] * inv * (448.f / 1e-4f) : (u[e] * 448.f) / amu;
    const uint32_t c = e4m3_code(q);
    if (e < 4)
      lo |= c << (8 * e);
    else
      hi |= c << (8 * (e - 4));
  }
  return make_uint2(lo, hi);
}

__device__ __forceinline__ void st_agent_u64(GLB void* p, uint2 v) {
  __hip_atomic_store((GLB uint64_t*)p, ((uint64_t)v.y << 32) | v.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- A0: add + RMSNorm + fp8 quant of token row m.WPay ------------------------
// Wave cw owns a quarter of the row's 128-column blocks: 16 lanes per block, 8
// elements per lane, up to GRP groups of four blocks per wave.  Every load of
// the wave's share (x, r and the norm weight) is issued at once; the wave's
// sum of squares goes through xsum, which returns the sum over the four waves
// (the same value, added in wave order, on every wave), and the codes are then
// formed from the values still in registers.  Outputs the residual sum in bf16,
// the norm output in fp32 (the gate's input) and the codes and scales (the
// other GEMMs' input).
constexpr int kA0Groups = 4;  // 16 blocks per wave: hidden up to 8192
template <class XSum>
__device__ inline void glm_a0_wave(const Meta& m, const Consts& c, int cw, const XSum& xsum,
                                   unsigned long long* tr = nullptr) {
  const int lane = lane_id(), row = m.w(WPay), H = c.H;
  const GLB uint16_t* x = (const GLB uint16_t*)m.q(GaX) + (size_t)row * H;
  const GLB uint16_t* r = (const GLB uint16_t*)m.q(GaR) + (size_t)row * H;
  const GLB uint16_t* w = (const GLB uint16_t*)m.q(GaNorm);
  const int nb = H / 128, per = (nb + kNW - 1) / kNW;
  const int b0 = cw * per, b1 = b0 + per < nb ? b0 + per : nb;
  u32x4 xv[kA0Groups], rv[kA0Groups], wv[kA0Groups];
  bool live[kA0Groups];
  int k0[kA0Groups];
#pragma unroll
  for (int gq = 0; gq < kA0Groups; ++gq) {
    const int blk = b0 + 4 * gq + (lane >> 4);
    live[gq] = blk < b1;
    k0[gq] = (live[gq] ? blk : 0) * 128 + (lane & 15) * 8;
    if (b0 + 4 * gq < b1) {
      xv[gq] = *(const GLB u32x4*)(x + k0[gq]);
      rv[gq] = *(const GLB u32x4*)(r + k0[gq]);
      wv[gq] = *(const GLB u32x4*)(w + k0[gq]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // one memory latency for all of them
  float h[kA0Groups][8];
  float ss = 0.f;
#pragma unroll
  for (int gq = 0; gq < kA0Groups; ++gq) {
    if (b0 + 4 * gq >= b1) continue;
    const uint32_t xw[4] = {xv[gq].x, xv[gq].y, xv[gq].z, xv[gq].w};
    const uint32_t rw[4] = {rv[gq].x, rv[gq].y, rv[gq].z, rv[gq].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[gq][2 * e] = bf16lo(xw[e]) + bf16lo(rw[e]);
      h[gq][2 * e + 1] = bf16hi(xw[e]) + bf16hi(rw[e]);
    }
    if (live[gq]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(h[gq][e], h[gq][e], ss);
    }
  }
  if (tr && lane == 0) tr[6] = now_ticks();
  const float inv = 1.f / sqrtf(xsum(wave_sum(ss)) / (float)H + c.eps);
  if (tr && lane == 0) tr[7] = now_ticks();
  GLB uint16_t* rout = (GLB uint16_t*)m.q(GaROut) + (size_t)row * H;
  GLB float* nout = (GLB float*)m.q(GaN) + (size_t)row * H;
  GLB uint8_t* codes = (GLB uint8_t*)m.q(GaA8) + (size_t)row * H;
  GLB float* scales = (GLB float*)m.q(GaAS) + (size_t)row * nb;
#pragma unroll
  for (int gq = 0; gq < kA0Groups; ++gq) {
    if (b0 + 4 * gq >= b1) continue;
    const uint32_t ww[4] = {wv[gq].x, wv[gq].y, wv[gq].z, wv[gq].w};
    float u[8], n[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[2 * e] = h[gq][2 * e] * bf16lo(ww[e]);
      u[2 * e + 1] = h[gq][2 * e + 1] * bf16hi(ww[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] = u[e] * inv;
    float sc;
    const uint2 q = glm_quant8(u, inv, &sc);
    if (live[gq]) {
      u32x4 hb;
      hb.x = (uint32_t)f2bf(h[gq][0]) | ((uint32_t)f2bf(h[gq][1]) << 16);
      hb.y = (uint32_t)f2bf(h[gq][2]) | ((uint32_t)f2bf(h[gq][3]) << 16);
      hb.z = (uint32_t)f2bf(h[gq][4]) | ((uint32_t)f2bf(h[gq][5]) << 16);
      hb.w = (uint32_t)f2bf(h[gq][6]) | ((uint32_t)f2bf(h[gq][7]) << 16);
      *(GLB u32x4*)(rout + k0[gq]) = hb;
      st_agent16(nout, (uint32_t)k0[gq] * 4, f32x4{n[0], n[1], n[2], n[3]});
      st_agent16(nout, (uint32_t)(k0[gq] + 4) * 4, f32x4{n[4], n[5], n[6], n[7]});
      st_agent_u64(codes + k0[gq], q);
      if ((lane & 15) == 0) st_agent(scales + (k0[gq] >> 7), sc);
    }
  }
}

// ---- q path: RMSNorm + requant of QKV-A's q columns, KV row ----------------------
// Waves 0..2 own a third of the q blocks each (up to QG groups of four blocks;
// their sums of squares are added through xsum, wave 3 adding zero); wave 3
// normalizes the kv columns, rotates the k_rope columns and writes the bf16 row
// [kv | k_rope] at the token's position of its request's cache.  Every load of a
// wave is issued before any is used.
constexpr int kQaGroups = 2;  // 8 blocks per wave: q_lora up to 3072
constexpr int kKvChunks = 2;  // 16-byte kv chunks per lane of wave 3: kv_lora up to 1024
template <int POL = 0, class XSum>
__device__ inline void glm_qan_wave(const Meta& m, const Consts& c, int cw, const XSum& xsum) {
  const int lane = lane_id(), row = m.w(WPay);
  const CohT<POL> ci((const GLB float*)m.q(QnIn) + (size_t)row * c.na);  // the row's QKV-A output
  if (cw < 3) {
    const int nb = c.ql / 128, per = (nb + 2) / 3;
    const int b0 = cw * per, b1 = b0 + per < nb ? b0 + per : nb;
    const GLB uint16_t* w = (const GLB uint16_t*)m.q(QnNorm);
    f32x4 x0[kQaGroups], x1[kQaGroups];
    u32x4 wv[kQaGroups];
    bool live[kQaGroups];
    int k0[kQaGroups];
#pragma unroll
    for (int gq = 0; gq < kQaGroups; ++gq) {
      const int blk = b0 + 4 * gq + (lane >> 4);
      live[gq] = blk < b1;
      k0[gq] = (live[gq] ? blk : 0) * 128 + (lane & 15) * 8;
      if (b0 + 4 * gq < b1) {
        x0[gq] = ci.f4((uint32_t)k0[gq] * 4);
        x1[gq] = ci.f4((uint32_t)(k0[gq] + 4) * 4);
        wv[gq] = *(const GLB u32x4*)(w + k0[gq]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    float ss = 0.f;
#pragma unroll
    for (int gq = 0; gq < kQaGroups; ++gq) {
      if (b0 + 4 * gq < b1 && live[gq]) {
        ss = fmaf(x0[gq].x, x0[gq].x, fmaf(x0[gq].y, x0[gq].y, fmaf(x0[gq].z, x0[gq].z, fmaf(x0[gq].w, x0[gq].w, ss))));
        ss = fmaf(x1[gq].x, x1[gq].x, fmaf(x1[gq].y, x1[gq].y, fmaf(x1[gq].z, x1[gq].z, fmaf(x1[gq].w, x1[gq].w, ss))));
      }
    }
    const float inv = 1.f / sqrtf(xsum(wave_sum(ss)) / (float)c.ql + c.eps);
    GLB uint8_t* codes = (GLB uint8_t*)m.q(QnA8) + (size_t)row * c.ql;
    GLB float* scales = (GLB float*)m.q(QnAS) + (size_t)row * nb;
#pragma unroll
    for (int gq = 0; gq < kQaGroups; ++gq) {
      if (b0 + 4 * gq >= b1) continue;
      const float u[8] = {x0[gq].x * bf16lo(wv[gq].x), x0[gq].y * bf16hi(wv[gq].x), x0[gq].z * bf16lo(wv[gq].y),
                          x0[gq].w * bf16hi(wv[gq].y), x1[gq].x * bf16lo(wv[gq].z), x1[gq].y * bf16hi(wv[gq].z),
                          x1[gq].z * bf16lo(wv[gq].w), x1[gq].w * bf16hi(wv[gq].w)};
      float sc;
      const uint2 q = glm_quant8(u, inv, &sc);
      if (live[gq]) {
        st_agent_u64(codes + k0[gq], q);
        if ((lane & 15) == 0) st_agent(scales + (k0[gq] >> 7), sc);
      }
    }
  } else {
    (void)xsum(0.f);  // wave 3 takes part in the exchange with nothing to add
    const GLB int* rows = (const GLB int*)m.q(QnRows);
    const GLB uint16_t* w = (const GLB uint16_t*)m.q(QnKvNorm);
    const int half = c.rd / 2, kr = c.ql + c.kl;  // kr: first k_rope column
    const int nch = c.kl / 8;                      // 8-element chunks of the kv columns
    f32x4 v0[kKvChunks], v1[kKvChunks];
    u32x4 wv[kKvChunks];
#pragma unroll
    for (int j = 0; j < kKvChunks; ++j) {
      const int ch = lane + 64 * j < nch ? lane + 64 * j : 0;
      v0[j] = ci.f4((uint32_t)(c.ql + ch * 8) * 4);
      v1[j] = ci.f4((uint32_t)(c.ql + ch * 8 + 4) * 4);
      wv[j] = *(const GLB u32x4*)(w + ch * 8);
    }
    const int pl = lane < half ? lane : 0;
    const float r0 = ci.f1((uint32_t)(kr + pl) * 4), r1 = ci.f1((uint32_t)(kr + pl + half) * 4);
    const GLB float* rope = (const GLB float*)m.q(QnRope) + ((size_t)row * half + pl) * 2;
    const float cs = rope[0], sn = rope[1];
    const int pos = rows[row], req = rows[c.B + row];
    __builtin_amdgcn_sched_barrier(0);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < kKvChunks; ++j) {
      if (lane + 64 * j < nch) {
        ss = fmaf(v0[j].x, v0[j].x, fmaf(v0[j].y, v0[j].y, fmaf(v0[j].z, v0[j].z, fmaf(v0[j].w, v0[j].w, ss))));
        ss = fmaf(v1[j].x, v1[j].x, fmaf(v1[j].y, v1[j].y, fmaf(v1[j].z, v1[j].z, fmaf(v1[j].w, v1[j].w, ss))));
      }
    }
    const float inv = 1.f / sqrtf(wave_sum(ss) / (float)c.kl + c.eps);
    GLB uint16_t* out = (GLB uint16_t*)m.q(QnKv) + ((size_t)req * c.cap + pos) * (c.kl + c.rd);
#pragma unroll
    for (int j = 0; j < kKvChunks; ++j) {
      if (lane + 64 * j < nch) {
        const int e0 = (lane + 64 * j) * 8;
        const float n8[8] = {v0[j].x * inv * bf16lo(wv[j].x), v0[j].y * inv * bf16hi(wv[j].x),
                             v0[j].z * inv * bf16lo(wv[j].y), v0[j].w * inv * bf16hi(wv[j].y),
                             v1[j].x * inv * bf16lo(wv[j].z), v1[j].y * inv * bf16hi(wv[j].z),
                             v1[j].z * inv * bf16lo(wv[j].w), v1[j].w * inv * bf16hi(wv[j].w)};
        u32x4 o;  // rows are (kv_lora + rope_dim) bf16 long, 16-byte aligned (checked on the host)
        o.x = (uint32_t)f2bf(n8[0]) | ((uint32_t)f2bf(n8[1]) << 16);
        o.y = (uint32_t)f2bf(n8[2]) | ((uint32_t)f2bf(n8[3]) << 16);
        o.z = (uint32_t)f2bf(n8[4]) | ((uint32_t)f2bf(n8[5]) << 16);
        o.w = (uint32_t)f2bf(n8[6]) | ((uint32_t)f2bf(n8[7]) << 16);
        *(GLB u32x4*)(out + e0) = o;
      }
    }
    if (lane < half) {
      out[c.kl + lane] = f2bf(r0 * cs - r1 * sn);
      out[c.kl + lane + half] = f2bf(r1 * cs + r0 * sn);
    }
  }
}

// ---- epilogue of an fp8 GEMM tile (storer wave) ---------------------------------
// Lane l: token b = l % 16, tile rows 4 (l / 16) + i.  The four waves' partial
// blocks are summed in wave order.  A RoPE-pair tile holds rows row0 + p (tile
// rows 0..7) and row1 + p (tile rows 8..15) for p < 8, partners in lanes l and
// l ^ 32; the rotation angle is that of rope frequency (row0 mod head_dim) -
// nope + p.
__device__ inline void glm_epilogue(const Meta& m, const Consts& c, const LDS float* part) {
  const int lane = lane_id(), b = lane & 15, q = lane >> 4;
  const int op = m.w(WOpcode), row0 = m.w(WPay), nrows = m.w(WPay + 1), row1 = m.w(WPay + 2);
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = (4 * q + i) * kMB + b;
    v[i] = ((part[k] + part[kMB * kMB + k]) + part[2 * kMB * kMB + k]) + part[3 * kMB * kMB + k];
  }
  const bool bok = b < c.B;
  if (row1 >= 0) {
    const int hd = c.nope + c.rd, half = c.rd / 2;
    const GLB float* rope = (const GLB float*)m.q(GmRope) + (size_t)(bok ? b : 0) * half * 2;
    GLB uint16_t* out = (GLB uint16_t*)m.q(GmOut) + (size_t)b * c.nq * hd;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float partner = __shfl_xor(v[i], 32, 64);
      const int tr = 4 * q + i;
      const int p = tr < 8 ? tr : tr - 8;
      const int f = row0 % hd - c.nope + p;
      const float cs = rope[2 * f], sn = rope[2 * f + 1];
      if (bok && p < nrows) {
        if (tr < 8)
          out[row0 + p] = f2bf(v[i] * cs - partner * sn);
        else
          out[row1 + p] = f2bf(v[i] * cs + partner * sn);
      }
    }
    return;
  }
  if (!bok) return;
  if (op == OpGGate) {
    // the K-split's partial block: [split][row tile][token][16 rows], four
    // consecutive rows of token b per lane (the reduce op adds the splits)
    const int Tg = (c.ng + kMB - 1) / kMB;
    const uint32_t at = (uint32_t)(((m.w(WGy) * Tg + m.w(WGx)) * kMB + b) * kMB + 4 * q) * 4;
    st_agent16((const GLB float*)m.q(GmOut), at, f32x4{v[0], v[1], v[2], v[3]});
    return;
  }
  if (op == OpGQkva && 4 * q + 3 < nrows) {
    // four consecutive outputs of token b in one 16-byte store (rows of
    // q_lora + kv_lora + rope_dim floats, a multiple of 4: checked on the host)
    st_agent16((const GLB float*)m.q(GmOut), (uint32_t)(b * c.na + row0 + 4 * q) * 4, f32x4{v[0], v[1], v[2], v[3]});
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = 4 * q + i;
    if (tr >= nrows) continue;
    const int n = row0 + tr;
    switch (op) {
      case OpGQkva:
        st_agent((GLB float*)m.q(GmOut) + (size_t)b * c.na + n, v[i]);
        break;
      case OpGIdxk: {
        const GLB int* rows = (const GLB int*)m.q(GmRows);
        const size_t at = ((size_t)rows[c.B + b] * c.cap + rows[b]) * c.nik + n;
        ((GLB uint16_t*)m.q(GmOut))[at] = f2bf(v[i]);
        break;
      }
      case OpGQkvb:
        ((GLB uint16_t*)m.q(GmOut))[(size_t)b * c.nq * (c.nope + c.rd) + n] = f2bf(v[i]);
        break;
      default:  // OpGIdxq
        ((GLB uint16_t*)m.q(GmOut))[(size_t)b * c.niq + n] = f2bf(v[i]);
        break;
    }
  }
}

// ---- head-gate reduce: the K-split partials of one row tile, in split order --------
// One wave: lane l holds token l % 16, rows 4 (l / 16) .. + 3; the splits'
// partials are loaded in batches of kGateRedBatch (one memory latency each)
// and added in split order.
constexpr int kMaxGateSplits = 16;
constexpr int kGateRedBatch = 4;
template <int POL = 0>
__device__ inline void glm_gate_red_wave(const Meta& m, const Consts& c, int cw) {
  if (cw != 0) return;
  const int lane = lane_id(), b = lane & 15, q = lane >> 4;
  const int row0 = m.w(WPay), GS = m.w(WPay + 2), x = m.w(WGx);
  const int Tg = (c.ng + kMB - 1) / kMB;
  const CohT<POL> cp((const GLB float*)m.q(GrPart));
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < GS; z0 += kGateRedBatch) {
    f32x4 pv[kGateRedBatch];
#pragma unroll
    for (int u = 0; u < kGateRedBatch; ++u) {
      const int z = z0 + u < GS ? z0 + u : z0;
      pv[u] = cp.f4((uint32_t)(((z * Tg + x) * kMB + b) * kMB + 4 * q) * 4);
    }
#pragma unroll
    for (int u = 0; u < kGateRedBatch; ++u)
      if (z0 + u < GS) acc += pv[u];
  }
  if (b < c.B) *(GLB f32x4*)((GLB float*)m.q(GrOut) + (size_t)b * c.ng + row0 + 4 * q) = acc;
}

}  // namespace mkd
