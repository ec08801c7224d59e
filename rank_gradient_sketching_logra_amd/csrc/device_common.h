// Device-side building blocks shared by the LoGRA kernels (gfx950 / CDNA4).
//
// - Philox4x64-10 and Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
//   Random Numbers: As Easy as 1, 2, 3", SC'11): the counter-based generators
//   that regenerate the Rademacher projection's signs and the
//   stochastic-rounding draws (4x32: two 32x32-bit products per round instead
//   of two 64x64-bit ones, about a quarter of the multiplies per bit) and the
//   Gaussian projection variant's entries (4x64).
// - bf16 rounding: nearest-even and deterministic stochastic rounding of an
//   fp32 value.  Stochastic rounding moves to the far bf16 neighbour with
//   probability equal to the fraction of the gap ("Randomized Gradient
//   Compression" blog, "How it works"); with a 16-bit draw u this is "add u
//   to the 16 discarded bits and truncate".
// - MFMA operand vector types for v_mfma_f32_32x32x16_bf16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logra {

// ----------------------------------------------------------------- Philox

// Multipliers and Weyl key increments of Philox4x64 (SC'11).
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

struct Philox4 {
  uint64_t w[4];
};

// Ten rounds.  Each round multiplies words 0 and 2 by the two constants,
// and the new counter is (hi(M1*x2)^x1^k0, lo(M1*x2), hi(M0*x0)^x3^k1,
// lo(M0*x0)); the key advances by the Weyl constants between rounds.
__device__ __forceinline__ Philox4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                                 uint64_t c3, uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t lo0 = c0 * kPhiloxM0;
    const uint64_t hi0 = __umul64hi(c0, kPhiloxM0);
    const uint64_t lo1 = c2 * kPhiloxM1;
    const uint64_t hi1 = __umul64hi(c2, kPhiloxM1);
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  Philox4 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// Key words of a projection: (seed, step << 32 | matrix_id).
struct KeyWords {
  uint64_t k0, k1;
};

// Four standard normal entries of the Gaussian projection variant, columns
// 4c .. 4c + 3 of row j: Box-Muller (Box and Muller, 1958) on the block with
// counter (j, c, 2, 0), uniforms u_i = ((w_i >> 11) + 1/2) 2^-53, pairs
// (u0, u1) and (u2, u3), cosine then sine; fp64.
__device__ __forceinline__ void gaussian_block(KeyWords key, uint64_t j, uint64_t c, double (&z)[4]) {
  const Philox4 p = philox4x64_10(j, c, 2, 0, key.k0, key.k1);
  double u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = ((double)(p.w[i] >> 11) + 0.5) * 0x1.0p-53;
  const double two_pi = 6.283185307179586476925286766559;
  const double rho0 = sqrt(-2.0 * log(u[0])), rho1 = sqrt(-2.0 * log(u[2]));
  z[0] = rho0 * cos(two_pi * u[1]);
  z[1] = rho0 * sin(two_pi * u[1]);
  z[2] = rho1 * cos(two_pi * u[3]);
  z[3] = rho1 * sin(two_pi * u[3]);
}

// Multipliers and Weyl key increments of Philox4x32 (SC'11).
constexpr uint32_t kPhilox32M0 = 0xD2511F53u;
constexpr uint32_t kPhilox32M1 = 0xCD9E8D57u;
constexpr uint32_t kPhilox32W0 = 0x9E3779B9u;
constexpr uint32_t kPhilox32W1 = 0xBB67AE85u;

struct Philox4x32 {
  uint32_t w[4];
};

// Ten rounds of the same structure on 32-bit words: each 32x32-bit product
// gives hi and lo in one multiply-add.
__device__ __forceinline__ Philox4x32 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                    uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)c0 * kPhilox32M0;
    const uint64_t p1 = (uint64_t)c2 * kPhilox32M1;
    c0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    c1 = (uint32_t)p1;
    c2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c3 = (uint32_t)p0;
    k0 += kPhilox32W0;
    k1 += kPhilox32W1;
  }
  Philox4x32 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// 256 sign bits of row j, columns [256*b, 256*b + 256) of sigma, as four
// 64-bit words: bit l & 255 (word (l & 255) >> 6, bit l & 63) set means -1.
// They are two Philox4x32-10 blocks, one per 128-column group c = l >> 7,
// with counter (c, j | 2^31, matrix_id, step) under key (seed lo, seed hi);
// column l is bit l & 31 of the block's word (l & 127) >> 5, so 64-bit word i
// is words 2(i & 1) (low half) and 2(i & 1) + 1 (high half) of block 2b + (i >> 1).
__device__ __forceinline__ Philox4 sigma_block(KeyWords key, uint64_t j, uint64_t b) {
  const uint32_t c1 = (uint32_t)j | 0x80000000u;
  const uint32_t mid = (uint32_t)key.k1, step = (uint32_t)(key.k1 >> 32);
  const uint32_t s0 = (uint32_t)key.k0, s1 = (uint32_t)(key.k0 >> 32);
  const Philox4x32 lo = philox4x32_10((uint32_t)(2 * b), c1, mid, step, s0, s1);
  const Philox4x32 hi = philox4x32_10((uint32_t)(2 * b + 1), c1, mid, step, s0, s1);
  Philox4 out;
  out.w[0] = (uint64_t)lo.w[0] | ((uint64_t)lo.w[1] << 32);
  out.w[1] = (uint64_t)lo.w[2] | ((uint64_t)lo.w[3] << 32);
  out.w[2] = (uint64_t)hi.w[0] | ((uint64_t)hi.w[1] << 32);
  out.w[3] = (uint64_t)hi.w[2] | ((uint64_t)hi.w[3] << 32);
  return out;
}

// 8 stochastic-rounding draws for flat elements [8*g, 8*g + 8) of the matrix
// whose key is (sr_seed, step << 32 | matrix_id): the Philox4x32-10 block
// with counter (g lo, g hi, matrix_id, step) under key (sr_seed lo, sr_seed
// hi); the draw of element e is bits [16*(e & 1), +16) of word (e & 7) >> 1.
__device__ __forceinline__ Philox4x32 sr_block(KeyWords key, uint64_t g) {
  return philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), (uint32_t)key.k1,
                       (uint32_t)(key.k1 >> 32), (uint32_t)key.k0, (uint32_t)(key.k0 >> 32));
}

__device__ __forceinline__ uint32_t sr_draw(const Philox4x32& p, uint64_t e) {
  // The word is picked by selects on register values, not by indexing: an
  // indexed pick (which the compiler also forms from selects of the array's
  // elements) puts the block in private or LDS memory and makes the kernel
  // wait for it.
  uint32_t w0 = p.w[0], w1 = p.w[1], w2 = p.w[2], w3 = p.w[3];
  asm("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
  const uint32_t i = (uint32_t)(e & 7) >> 1;
  const uint32_t w = (i & 2) ? ((i & 1) ? w3 : w2) : ((i & 1) ? w1 : w0);
  return (w >> (16 * (uint32_t)(e & 1))) & 0xFFFFu;
}

// ------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Nearest-even rounding of an fp32 value to bf16 (bit pattern in the low 16
// bits).  Adding 0x7FFF plus the lowest kept bit to the pattern carries into
// the kept bits exactly when the discarded part is above half, or exactly
// half with an odd kept part.  Overflow lands on infinity.  NaN maps to a
// quiet NaN of the same sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) & 0x8000u) | 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Stochastic rounding with a 16-bit draw u: the discarded 16 bits are the
// position inside the gap in units of 2^-16, so adding u and truncating
// moves away from zero exactly when floor(fraction * 2^16) + u >= 2^16.
// Infinity and NaN round to nearest.
__device__ __forceinline__ uint32_t f32_to_bf16_sr(float f, uint32_t u16) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return f32_to_bf16_rne(f);
  return (u + u16) >> 16;
}

// --------------------------------------------------------------- MFMA types

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Eight bf16 values +-1 (an MFMA operand of signs) in a paired order: dword
// p takes its low element's sign from bit 15 - p of w and its high element's
// from bit 31 - p (bit set -> -1).  Two VALU operations per dword.
// (x & m) | c is one v_and_or_b32 only when m and c sit in registers (that
// encoding carries no two literals), so the constants are passed through an
// empty asm statement that makes them opaque.  The instruction itself is left
// to the compiler: it then knows a VALU op writes the register and inserts the
// wait states the matrix core needs before reading it as an operand (an
// and_or written in inline assembly is invisible to that hazard check, and the
// MFMA read a stale register).
__device__ __forceinline__ u32x4 expand_sign_pairs(uint32_t w) {
  uint32_t m = 0x80008000u, one = 0x3F803F80u;
  asm("" : "+v"(m), "+v"(one));
  u32x4 v;
  v[0] = (w & m) | one;
  v[1] = ((w << 1) & m) | one;
  v[2] = ((w << 2) & m) | one;
  v[3] = ((w << 3) & m) | one;
  return v;
}

// Split an fp32 value into bf16 hi + bf16 lo with hi = RNE(x) and
// lo = RNE(x - hi); hi + lo carries ~16 significant bits.
__device__ __forceinline__ void split_hi_lo(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_rne(x);
  lo = f32_to_bf16_rne(x - bf16_bits_to_f32(hi));
}

}  // namespace logra
