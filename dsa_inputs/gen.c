/*
 * Seeded synthetic inputs for the DeepSeek Sparse Attention hot path.
 *
 * This file draws random tensors and nothing else: it holds none of the
 * method's arithmetic (no scoring, selection or attention).  Both the CPU
 * oracle and the GPU path receive the bytes it writes, so the two are compared
 * on identical inputs.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-style: the draw for element i
 * of a tensor is the (i+1)-th SplitMix64 output from a state derived from
 * (seed, tensor id).  Any element range can therefore be produced on its own,
 * which lets a test build single query rows of a very large workload.
 *
 * Value recipes (the workload description of the DSA prefill/decode configs):
 *   - FP8 grid:   v = (u - 16) / 4 with u uniform on {0..32}, i.e. the 33
 *                 points {-4, -3.75, ..., 4}, stored as OCP e4m3fn bytes
 *                 (every grid point is exactly representable).
 *   - fp32 grid:  v = lo + step * u with u uniform on {0..npoints-1}.
 *   - bf16 N(0,1): Box-Muller in double precision from two 53-bit uniforms,
 *                 rounded to fp32 and then to bf16 (round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM64_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* State for one tensor of one workload. */
static inline uint64_t stream_state(uint64_t seed, uint64_t tensor_id) {
  return sm64_mix(sm64_mix(seed + SM64_GAMMA) ^ (tensor_id * 0xD1B54A32D192ED03ULL));
}

/* (i+1)-th SplitMix64 output from `state`. */
static inline uint64_t draw(uint64_t state, uint64_t i) {
  return sm64_mix(state + (i + 1) * SM64_GAMMA);
}

/* Uniform integer on {0..m-1} from the high 32 bits (multiply-shift). */
static inline uint32_t uniform_below(uint64_t h, uint32_t m) {
  return (uint32_t)(((h >> 32) * (uint64_t)m) >> 32);
}

/* Encode an exactly representable value as an OCP e4m3fn byte.
 * Returns 0xFF (a NaN code) when the value is not representable. */
static uint8_t encode_e4m3_exact(double v) {
  uint8_t sign = 0;
  if (v < 0) { sign = 0x80; v = -v; }
  if (v == 0.0) return sign;
  for (int e = 0; e < 16; ++e) {
    for (int m = 0; m < 8; ++m) {
      if (e == 15 && m == 7) continue;
      double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
      if (mag == v) return (uint8_t)(sign | (e << 3) | m);
    }
  }
  return 0xFF;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* q_I / k_I: the 33-point 0.25-step grid on [-4, 4], as e4m3fn bytes.
 * Writes elements [offset, offset + n) of the tensor. */
void dsa_gen_e4m3_grid(uint64_t seed, uint64_t tensor_id, int64_t offset, int64_t n,
                       uint8_t* out) {
  uint8_t table[33];
  for (int u = 0; u < 33; ++u) table[u] = encode_e4m3_exact((u - 16) / 4.0);
  const uint64_t st = stream_state(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = table[uniform_below(draw(st, (uint64_t)(offset + i)), 33)];
}

/* Real-valued grid lo + step * u, u uniform on {0..npoints-1}, as fp32. */
void dsa_gen_f32_grid(uint64_t seed, uint64_t tensor_id, int64_t offset, int64_t n,
                      int32_t npoints, double lo, double step, float* out) {
  const uint64_t st = stream_state(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(lo + step * (double)uniform_below(draw(st, (uint64_t)(offset + i)), (uint32_t)npoints));
}

/* N(0,1) as bf16 bits.  Element 2p and 2p+1 are the cosine and sine outputs of
 * one Box-Muller pair built from draws 2p and 2p+1. */
void dsa_gen_bf16_normal(uint64_t seed, uint64_t tensor_id, int64_t offset, int64_t n,
                         uint16_t* out) {
  const uint64_t st = stream_state(seed, tensor_id);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t e = (uint64_t)(offset + i);
    const uint64_t p = e >> 1;
    const double u1 = ((double)(draw(st, 2 * p) >> 11) + 1.0) * 0x1.0p-53; /* (0, 1] */
    const double u2 = (double)(draw(st, 2 * p + 1) >> 11) * 0x1.0p-53;     /* [0, 1) */
    const double r = sqrt(-2.0 * log(u1));
    const double z = (e & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
    out[i] = f32_to_bf16_rne((float)z);
  }
}
