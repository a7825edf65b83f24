/* Seeded synthetic input generator, shared by the CPU oracle and the HIP path.
 *
 * It holds none of the decode step's arithmetic: only a counter-based random
 * stream and the bit-level conversion of the drawn values to the storage
 * formats the inputs use (bf16).
 *
 * Stream definition (stable across machines and thread counts):
 *   mix(x)      = SplitMix64 output function applied to x + 0x9E3779B97F4A7C15
 *                 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *                 generators", OOPSLA 2014; constants from Vigna's public
 *                 reference implementation).
 *   key(s, t)   = mix(mix(s) ^ (t * 0xD1B54A32D192ED03))   seed s, tensor id t
 *   word(k, i)  = mix(k + i)
 *   normal i    : r1 = word(k, 2i), r2 = word(k, 2i+1),
 *                 u1 = ((r1 >> 11) + 1) * 2^-53 in (0,1], u2 = (r2 >> 11) * 2^-53,
 *                 z  = sqrt(-2 ln u1) * cos(2 pi u2)            (Box-Muller, fp64)
 *                 value = mean + sigma * z, rounded to fp32, then fp32 -> bf16
 *                 round-to-nearest-even on the bit pattern.
 *   uniform int : lo + word(k, i) mod (hi - lo + 1)
 *   fp8 weights : w[n][k] = fp32(sigma * normal(n * K + k)); per 128 x 128
 *                 block (row block n / 128, column block k / 128) the fp32 scale
 *                 is amax / 448 (1 when the block is all zero) and the stored
 *                 byte is the OCP FP8 E4M3 (e4m3fn) code of w / scale, rounded
 *                 to nearest even and saturated to +-448.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

static inline uint64_t mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static inline uint64_t key_of(uint64_t seed, uint64_t tid) {
  return mix(mix(seed) ^ (tid * 0xD1B54A32D192ED03ull));
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0x7FC0; /* NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline double normal_at(uint64_t k, uint64_t i) {
  uint64_t r1 = mix(k + 2 * i), r2 = mix(k + 2 * i + 1);
  double u1 = (double)((r1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(r2 >> 11) * 0x1.0p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

/* out[j] = bf16(mean + sigma * N_{offset+j}) for j in [0, n) */
void synth_normal_bf16(uint64_t seed, uint64_t tid, double mean, double sigma,
                       uint64_t offset, uint64_t n, uint16_t* out) {
  uint64_t k = key_of(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = f32_to_bf16_rne((float)(mean + sigma * normal_at(k, offset + (uint64_t)j)));
}

/* Strided variant for blocks of rows: element (r, c) of an [rows, cols] block
 * takes stream index base + r * row_stride + c. */
void synth_normal_bf16_2d(uint64_t seed, uint64_t tid, double mean, double sigma,
                          uint64_t base, uint64_t row_stride, uint64_t rows,
                          uint64_t cols, uint16_t* out) {
  uint64_t k = key_of(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < (int64_t)rows; ++r)
    for (uint64_t c = 0; c < cols; ++c)
      out[(uint64_t)r * cols + c] =
          f32_to_bf16_rne((float)(mean + sigma * normal_at(k, base + (uint64_t)r * row_stride + c)));
}

/* fp64 normals, for inputs that are consumed before any storage rounding. */
void synth_normal_f64(uint64_t seed, uint64_t tid, double mean, double sigma,
                      uint64_t offset, uint64_t n, double* out) {
  uint64_t k = key_of(seed, tid);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = mean + sigma * normal_at(k, offset + (uint64_t)j);
}

void synth_uniform_i32(uint64_t seed, uint64_t tid, int64_t lo, int64_t hi, uint64_t n, int32_t* out) {
  uint64_t k = key_of(seed, tid);
  uint64_t span = (uint64_t)(hi - lo + 1);
  for (uint64_t j = 0; j < n; ++j) out[j] = (int32_t)(lo + (int64_t)(mix(k + j) % span));
}

void synth_fill_u16(uint16_t v, uint64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) out[j] = v;
}

uint64_t synth_mix(uint64_t x) { return mix(x); }
uint16_t synth_f32_to_bf16(float f) { return f32_to_bf16_rne(f); }

/* OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * no infinities; S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8; smallest
 * normal 2^-6; subnormals m * 2^-9).  Round to nearest even, saturate. */
static uint8_t e4m3_code(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0x1.0p-6) { /* subnormal range: multiples of 2^-9 (8 * 2^-9 is the smallest normal) */
    double m = nearbyint(a * 512.0);
    return sign | (uint8_t)m;
  }
  int ex;
  double f = frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
  int E = ex - 1;           /* a = (2f) * 2^E, 2f in [1, 2) */
  double q = nearbyint((2.0 * f - 1.0) * 8.0);
  if (q == 8.0) { q = 0.0; ++E; }
  if (E > 8 || (E == 8 && q == 7.0)) return sign | 0x7E;
  return sign | (uint8_t)(((E + 7) << 3) | (int)q);
}

/* [N, K] fp8 weights and [ceil(N / 128), K / 128] fp32 block scales (K % 128 == 0). */
void synth_fp8_weights(uint64_t seed, uint64_t tid, double sigma, uint64_t N, uint64_t K,
                       uint8_t* codes, float* scales) {
  uint64_t k = key_of(seed, tid);
  uint64_t NB = (N + 127) / 128, KB = K / 128;
#pragma omp parallel for schedule(static)
  for (int64_t bb = 0; bb < (int64_t)(NB * KB); ++bb) {
    uint64_t nb = (uint64_t)bb / KB, kb = (uint64_t)bb % KB;
    uint64_t n1 = (nb + 1) * 128 < N ? (nb + 1) * 128 : N;
    float amax = 0.f;
    for (uint64_t n = nb * 128; n < n1; ++n)
      for (uint64_t c = kb * 128; c < kb * 128 + 128; ++c) {
        float w = (float)(sigma * normal_at(k, n * K + c));
        float aw = fabsf(w);
        if (aw > amax) amax = aw;
      }
    float sc = amax > 0.f ? amax / 448.f : 1.f;
    scales[bb] = sc;
    for (uint64_t n = nb * 128; n < n1; ++n)
      for (uint64_t c = kb * 128; c < kb * 128 + 128; ++c) {
        float w = (float)(sigma * normal_at(k, n * K + c));
        codes[n * K + c] = e4m3_code((double)(w / sc));
      }
  }
}

uint8_t synth_e4m3_code(double v) { return e4m3_code(v); }
