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
__device__ inline void glm_gemm_wave(const Src& src, const Meta& m, const Consts& c, int cw, LDS float* part) {
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
    // the gate reads the unquantized fp32 norm output: bf16 high and low parts
    // against the exactly converted weights, 4 k-steps of 8 per lane per block
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    const CohT<POL> cx((const GLB float*)m.q(GmAF));
    const uint32_t xo = (uint32_t)(bb * K) * 4;
    for (int kb = kb0; kb < kb1; ++kb) {
      const int ko = kb * 128 + g * 32;
      const uint4 w0 = src.ld16(seg, rr * K + ko), w1 = src.ld16(seg, rr * K + ko + 16);
      const uint32_t wd[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      f32x4 blk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x4 x0 = cx.f4(xo + (uint32_t)(ko + ks * 8) * 4);
        const f32x4 x1 = cx.f4(xo + (uint32_t)(ko + ks * 8 + 4) * 4);
        const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        bf16x8 av, hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t code = (wd[2 * ks + e / 4] >> (8 * (e & 3))) & 0xFFu;
          av[e] = __builtin_bit_cast(__bf16, (uint16_t)e4m3_to_bf16(code));
          const __bf16 h = (__bf16)v[e];
          hi[e] = h;
          lo[e] = (__bf16)(v[e] - (float)h);
        }
        blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, hi, blk, 0, 0, 0);
        blk = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, lo, blk, 0, 0, 0);
      }
      const float sc = ws[kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(blk[i], sc, acc[i]);
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
// Every wave sums the squares of the whole row (the row is 2 x hidden bf16, read
// once from memory and then from the cache); wave cw then finishes its quarter
// of the 128-column blocks: 16 lanes per block, 8 elements per lane.  Outputs
// the residual sum in bf16, the norm output in fp32 (the gate's input) and the
// codes and scales (the other GEMMs' input).
__device__ inline void glm_a0_wave(const Meta& m, const Consts& c, int cw) {
  const int lane = lane_id(), row = m.w(WPay), H = c.H;
  const GLB uint16_t* x = (const GLB uint16_t*)m.q(GaX) + (size_t)row * H;
  const GLB uint16_t* r = (const GLB uint16_t*)m.q(GaR) + (size_t)row * H;
  const int nch = H / 8;
  float ss = 0.f;
  for (int j0 = 0; j0 < nch; j0 += 4 * 64) {
    u32x4 xv[4], rv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * 64 + lane;
      const int jj = j < nch ? j : 0;
      xv[u] = *(const GLB u32x4*)(x + jj * 8);
      rv[u] = *(const GLB u32x4*)(r + jj * 8);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (j0 + u * 64 + lane < nch) {
        const uint32_t xw[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w}, rw[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float h0 = bf16lo(xw[e]) + bf16lo(rw[e]), h1 = bf16hi(xw[e]) + bf16hi(rw[e]);
          ss = fmaf(h0, h0, ss);
          ss = fmaf(h1, h1, ss);
        }
      }
    }
  }
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss / (float)H + c.eps);
  const int nb = H / 128, per = (nb + kNW - 1) / kNW;
  const int b0 = cw * per, b1 = b0 + per < nb ? b0 + per : nb;
  const GLB uint16_t* w = (const GLB uint16_t*)m.q(GaNorm);
  GLB uint16_t* rout = (GLB uint16_t*)m.q(GaROut) + (size_t)row * H;
  GLB float* nout = (GLB float*)m.q(GaN) + (size_t)row * H;
  GLB uint8_t* codes = (GLB uint8_t*)m.q(GaA8) + (size_t)row * H;
  GLB float* scales = (GLB float*)m.q(GaAS) + (size_t)row * nb;
  for (int bq = b0; bq < b1; bq += 4) {
    const int blk = bq + (lane >> 4);
    const bool live = blk < b1;
    const int k0 = (live ? blk : b0) * 128 + (lane & 15) * 8;
    const u32x4 xv = *(const GLB u32x4*)(x + k0), rv = *(const GLB u32x4*)(r + k0), wv = *(const GLB u32x4*)(w + k0);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, rw[4] = {rv.x, rv.y, rv.z, rv.w}, ww[4] = {wv.x, wv.y, wv.z, wv.w};
    float h[8], u[8], n[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[2 * e] = bf16lo(xw[e]) + bf16lo(rw[e]);
      h[2 * e + 1] = bf16hi(xw[e]) + bf16hi(rw[e]);
      u[2 * e] = h[2 * e] * bf16lo(ww[e]);
      u[2 * e + 1] = h[2 * e + 1] * bf16hi(ww[e]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) n[e] = u[e] * inv;
    float sc;
    const uint2 q = glm_quant8(u, inv, &sc);
    if (live) {
      u32x4 hb;
      hb.x = (uint32_t)f2bf(h[0]) | ((uint32_t)f2bf(h[1]) << 16);
      hb.y = (uint32_t)f2bf(h[2]) | ((uint32_t)f2bf(h[3]) << 16);
      hb.z = (uint32_t)f2bf(h[4]) | ((uint32_t)f2bf(h[5]) << 16);
      hb.w = (uint32_t)f2bf(h[6]) | ((uint32_t)f2bf(h[7]) << 16);
      *(GLB u32x4*)(rout + k0) = hb;
#pragma unroll
      for (int e = 0; e < 8; ++e) st_agent(nout + k0 + e, n[e]);
      st_agent_u64(codes + k0, q);
      if ((lane & 15) == 0) st_agent(scales + blk, sc);
    }
  }
}

// ---- q path: RMSNorm + requant of QKV-A's q columns, KV row ----------------------
// Waves 0..2 share the q blocks (each sums the squares of all q columns); wave 3
// normalizes the kv columns, rotates the k_rope columns and writes the bf16 row
// [kv | k_rope] at the token's position of its request's cache.
template <int POL = 0>
__device__ inline void glm_qan_wave(const Meta& m, const Consts& c, int cw) {
  const int lane = lane_id(), row = m.w(WPay);
  const CohT<POL> ci((const GLB float*)m.q(QnIn) + (size_t)row * c.na);  // the row's QKV-A output
  auto sumsq = [&](int e0, int n) {  // elements e0 .. e0 + n - 1, n a multiple of 4
    float ss = 0.f;
    for (int j = lane; j < n / 4; j += 64) {
      const f32x4 v = ci.f4((uint32_t)(e0 + 4 * j) * 4);
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, fmaf(v.z, v.z, fmaf(v.w, v.w, ss))));
    }
    return wave_sum(ss);
  };
  if (cw < 3) {
    const float inv = 1.f / sqrtf(sumsq(0, c.ql) / (float)c.ql + c.eps);
    const int nb = c.ql / 128, per = (nb + 2) / 3;
    const int b0 = cw * per, b1 = b0 + per < nb ? b0 + per : nb;
    const GLB uint16_t* w = (const GLB uint16_t*)m.q(QnNorm);
    GLB uint8_t* codes = (GLB uint8_t*)m.q(QnA8) + (size_t)row * c.ql;
    GLB float* scales = (GLB float*)m.q(QnAS) + (size_t)row * nb;
    for (int bq = b0; bq < b1; bq += 4) {
      const int blk = bq + (lane >> 4);
      const bool live = blk < b1;
      const int k0 = (live ? blk : b0) * 128 + (lane & 15) * 8;
      const f32x4 x0 = ci.f4((uint32_t)k0 * 4), x1 = ci.f4((uint32_t)(k0 + 4) * 4);
      const u32x4 wv = *(const GLB u32x4*)(w + k0);
      const float u[8] = {x0.x * bf16lo(wv.x), x0.y * bf16hi(wv.x), x0.z * bf16lo(wv.y), x0.w * bf16hi(wv.y),
                          x1.x * bf16lo(wv.z), x1.y * bf16hi(wv.z), x1.z * bf16lo(wv.w), x1.w * bf16hi(wv.w)};
      float sc;
      const uint2 q = glm_quant8(u, inv, &sc);
      if (live) {
        st_agent_u64(codes + k0, q);
        if ((lane & 15) == 0) st_agent(scales + blk, sc);
      }
    }
  } else {
    const float inv = 1.f / sqrtf(sumsq(c.ql, c.kl) / (float)c.kl + c.eps);
    const GLB int* rows = (const GLB int*)m.q(QnRows);
    const int pos = rows[row], req = rows[c.B + row];
    GLB uint16_t* out = (GLB uint16_t*)m.q(QnKv) + ((size_t)req * c.cap + pos) * (c.kl + c.rd);
    const GLB uint16_t* w = (const GLB uint16_t*)m.q(QnKvNorm);
    for (int j = lane; j < c.kl; j += 64) out[j] = f2bf(ci.f1((uint32_t)(c.ql + j) * 4) * inv * bf16f(w[j]));
    const int half = c.rd / 2;
    if (lane < half) {
      const GLB float* rope = (const GLB float*)m.q(QnRope) + ((size_t)row * half + lane) * 2;
      const int kr = c.ql + c.kl;  // first k_rope column
      const float cs = rope[0], sn = rope[1];
      const float x0 = ci.f1((uint32_t)(kr + lane) * 4), x1 = ci.f1((uint32_t)(kr + lane + half) * 4);
      out[c.kl + lane] = f2bf(x0 * cs - x1 * sn);
      out[c.kl + lane + half] = f2bf(x1 * cs + x0 * sn);
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = 4 * q + i;
    if (tr >= nrows) continue;
    const int n = row0 + tr;
    switch (op) {
      case OpGQkva:
        st_agent((GLB float*)m.q(GmOut) + (size_t)b * c.na + n, v[i]);
        break;
      case OpGGate:
        ((GLB float*)m.q(GmOut))[(size_t)b * c.ng + n] = v[i];
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

}  // namespace mkd
