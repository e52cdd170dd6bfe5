// Device-side modular arithmetic for 64-bit RNS words on gfx950.
//
// Moduli are primes below 2^62 (54-bit ciphertext primes and 60-bit special
// primes in the benchmark parameter sets).  gfx950 has no 64x64-bit
// multiplier; every product is built from v_mad_u64_u32 (32x32+64 -> 64),
// which measures at close to full VALU rate on this chip, so the cost of an
// operation is essentially its instruction count.  The routines below are
// written so the compiler emits short mad chains:
//
//   mul_shoup      a*w mod q for a constant w with precomputed
//                  w' = floor(w*2^64/q) (Shoup's method).  Works for any
//                  64-bit a and returns a value in [0, 2q) -- no final
//                  correction, so callers stay lazy.
//   reduce_2q      [0, 2q) -> [0, q)
//   reduce64       any 64-bit value -> [0, q), using floor(2^64/q).
//   reduce_hi      partial reduction with a quotient from the high word
//                  (one 32-bit multiply-high), for q > 2^33.
//   U128 / mac     exact 128-bit accumulation of 64x64 products and one
//                  Barrett-style reduction per output.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace ckks {

struct U128 {
  uint64_t lo, hi;
};

__device__ __forceinline__ uint64_t mulhi64(uint64_t a, uint64_t b) { return __umul64hi(a, b); }

// Shoup: r = a*w - floor(a*w'/2^64)*q, in [0, 2q) for every a < 2^64.
__device__ __forceinline__ uint64_t mul_shoup(uint64_t a, uint64_t w, uint64_t wp, uint64_t q) {
  uint64_t qh = mulhi64(a, wp);
  return a * w - qh * q;
}

__device__ __forceinline__ uint64_t mad64(uint32_t a, uint32_t b, uint64_t c) { return (uint64_t)a * b + c; }

// Shoup with an approximate quotient: the high product a*w' is taken from
// the three upper 32x32 partial products only (the low one and the carries out
// of the discarded low halves are dropped), so the quotient is at most 2 below
// floor(a*w'/2^64) and the result lies in [0, 4q) for every a < 2^64.
// 3 v_mad/v_mul_hi for the quotient instead of 4 plus carry handling.
// The remainder a*w - qh*q is formed as lo64(a*w + qh*(2^64 - q)) with the two
// low 32x32 products chained through one 64-bit accumulator and the four
// cross products folded into its high word.
__device__ __forceinline__ uint64_t mul_shoup_lazy(uint64_t a, uint64_t w, uint64_t wp, uint64_t q) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t p0 = (uint32_t)wp, p1 = (uint32_t)(wp >> 32);
  // qh = a1 p1 + hi(a0 p1) + hi(a1 p0): drops a0 p0 and the low halves of the
  // two middle products, so it is at most 2 below floor(a w' / 2^64)
  const uint64_t s = (uint64_t)__umulhi(a0, p1) + (uint64_t)__umulhi(a1, p0);
  const uint64_t qh = mad64(a1, p1, s);
  const uint64_t nq = 0 - q;
  const uint32_t q0 = (uint32_t)qh, q1 = (uint32_t)(qh >> 32);
  const uint32_t w0 = (uint32_t)w, w1 = (uint32_t)(w >> 32);
  const uint32_t n0 = (uint32_t)nq, n1 = (uint32_t)(nq >> 32);
  uint64_t r = mad64(a0, w0, 0);
  r = mad64(q0, n0, r);  // modulo 2^64
  const uint32_t h = (uint32_t)(r >> 32) + a0 * w1 + a1 * w0 + q0 * n1 + q1 * n0;
  return ((uint64_t)h << 32) | (uint32_t)r;
}

__device__ __forceinline__ uint64_t reduce_2q(uint64_t a, uint64_t q) { return a >= q ? a - q : a; }

// The two halves of a 64-bit word as opaque 32-bit values.  In some kernels
// the compiler folds the partial products of mul_shoup_lazy back into a
// 64x64-bit multiply and lowers that as a longer multiply-add chain (about
// twice the instructions of the split form); taking the halves through an
// empty asm statement keeps the split form.  No instruction is emitted.
__device__ __forceinline__ void split_opaque(uint64_t a, uint32_t& lo, uint32_t& hi) {
  lo = (uint32_t)a;
  hi = (uint32_t)(a >> 32);
  asm("" : "+v"(lo), "+v"(hi));
}

// mul_shoup_lazy with both multiplicands split opaquely (same result).
__device__ __forceinline__ uint64_t mul_shoup_lazy_split(uint64_t a, uint64_t w, uint64_t wp, uint64_t q) {
  uint32_t a0, a1;
  split_opaque(a, a0, a1);
  const uint32_t p0 = (uint32_t)wp, p1 = (uint32_t)(wp >> 32);
  const uint64_t s = (uint64_t)__umulhi(a0, p1) + (uint64_t)__umulhi(a1, p0);
  const uint64_t qh = mad64(a1, p1, s);
  const uint64_t nq = 0 - q;
  uint32_t q0, q1;
  split_opaque(qh, q0, q1);
  const uint32_t w0 = (uint32_t)w, w1 = (uint32_t)(w >> 32);
  const uint32_t n0 = (uint32_t)nq, n1 = (uint32_t)(nq >> 32);
  uint64_t r = mad64(a0, w0, 0);
  r = mad64(q0, n0, r);
  const uint32_t h = (uint32_t)(r >> 32) + a0 * w1 + a1 * w0 + q0 * n1 + q1 * n0;
  return ((uint64_t)h << 32) | (uint32_t)r;
}

// [0, 4q) -> [0, q)
__device__ __forceinline__ uint64_t reduce_4q(uint64_t a, uint64_t q) {
  a = a >= 2 * q ? a - 2 * q : a;
  return a >= q ? a - q : a;
}

// a mod q for any 64-bit a, given inv1 = floor(2^64 / q).
__device__ __forceinline__ uint64_t reduce64(uint64_t a, uint64_t q, uint64_t inv1) {
  uint64_t r = a - mulhi64(a, inv1) * q;  // Shoup with w = 1: r in [0, 2q)
  return reduce_2q(r, q);
}

// For 2^33 < q (so m = floor(2^64/q) < 2^31): with h = floor(a / 2^32), the
// estimate e = floor(h m / 2^32) never exceeds a/q and falls short of it by
// less than 2^32/q + h/2^32 + 1, so a - e q lies in [0, 2.5q) for any 64-bit
// a and in [0, 2q) for a < 2^63.
__device__ __forceinline__ uint64_t reduce_hi(uint64_t a, uint64_t q, uint32_t m) {
  const uint32_t e = __umulhi((uint32_t)(a >> 32), m);
  return a - (uint64_t)e * q;
}
constexpr uint64_t kReduceHiMin = 1ull << 33;  // reduce_hi needs q above this

__device__ __forceinline__ U128 mul_wide(uint64_t a, uint64_t b) {
  U128 r;
  r.lo = a * b;
  r.hi = mulhi64(a, b);
  return r;
}

__device__ __forceinline__ void mac(U128& acc, uint64_t a, uint64_t b) {
  uint64_t lo = a * b;
  uint64_t hi = mulhi64(a, b);
  acc.lo += lo;
  acc.hi += hi + (acc.lo < lo ? 1 : 0);
}

// x mod q for a 128-bit x with x.hi < 2^63, given r64 = 2^64 mod q with its
// Shoup quotient r64p and inv1 = floor(2^64/q):
//   x = hi*2^64 + lo = hi*r64 + lo (mod q).
__device__ __forceinline__ uint64_t reduce128(U128 x, uint64_t q, uint64_t r64, uint64_t r64p, uint64_t inv1) {
  uint64_t a = mul_shoup(x.hi, r64, r64p, q);  // [0, 2q)
  uint64_t b = x.lo - mulhi64(x.lo, inv1) * q;  // [0, 2q)
  uint64_t s = a + b;                             // [0, 4q), q < 2^62
  s = s >= 2 * q ? s - 2 * q : s;
  return reduce_2q(s, q);
}

// Montgomery product a*b*2^-64 mod m for odd m < 2^63, mp = -m^-1 mod 2^64.
// P + u*m with u = lo(P)*mp is divisible by 2^64 and its low words cancel,
// so the carry out of the low half is (lo(P) != 0).  The result is below
// a*b/2^64 + m, so it lies in [0, 2m) whenever b < m, for ANY 64-bit a (the
// key-switch inner product multiplies lazy NTT outputs, up to 70q, by
// canonical key words).
__device__ __forceinline__ uint64_t mont_mul_lazy(uint64_t a, uint64_t b, uint64_t m, uint64_t mp) {
  const uint64_t lo = a * b;
  const uint64_t hi = mulhi64(a, b);
  const uint64_t u = lo * mp;
  return hi + mulhi64(u, m) + (lo != 0 ? 1 : 0);
}

// Lazy Montgomery products are below 2m; a running sum reduced to [0, m)
// after every k products stays below (2k + 1) m < 2^64 for k = 4 when
// m < 2^60, 3 when m < 2^61 and 1 when m < 2^62.
__host__ __device__ inline int mont_fold(uint64_t m) {
  return m < (1ull << 60) ? 4 : m < (1ull << 61) ? 3 : 1;
}

// ---------------------------------------------------------------------------
// Exact dot products of residues below 2^60 without carry chains.
// Each operand is split into 30-bit halves (v = vh*2^30 + vl); a product then
// has three column terms that are accumulated separately in 64-bit registers:
//   a0 = sum vl*cl,  a1 = sum (vl*ch + vh*cl),  a2 = sum vh*ch,
// every partial product is below 2^60, so up to 8 terms never overflow (a1
// holds 2 products per term).  One v_mad_u64_u32 per partial product.
struct Acc3 {
  uint64_t a0, a1, a2;
};

__device__ __forceinline__ uint32_t lo30(uint64_t v) { return (uint32_t)v & 0x3fffffffu; }
__device__ __forceinline__ uint32_t hi30(uint64_t v) { return (uint32_t)(v >> 30); }

__device__ __forceinline__ void acc3_mac(Acc3& A, uint32_t xl, uint32_t xh, uint32_t cl, uint32_t ch) {
  A.a0 = mad64(xl, cl, A.a0);
  A.a1 = mad64(xl, ch, A.a1);
  A.a1 = mad64(xh, cl, A.a1);
  A.a2 = mad64(xh, ch, A.a2);
}

// a0 + a1*2^30 + a2*2^60 as a 128-bit value (a0 < 2^63, a1 < 2^64, a2 < 2^63).
__device__ __forceinline__ U128 acc3_value(const Acc3& A) {
  U128 r;
  uint64_t t = A.a1 << 30;
  uint64_t lo = A.a0 + t;
  uint64_t hi = (A.a1 >> 34) + (lo < t ? 1 : 0);
  t = A.a2 << 60;
  r.lo = lo + t;
  r.hi = hi + (A.a2 >> 4) + (r.lo < t ? 1 : 0);
  return r;
}

// A value congruent to x mod q in [0, 6q), for x.hi < 2^64, using the
// approximate Shoup product for the high word: hi*2^64 = hi*r64 (mod q).
__device__ __forceinline__ uint64_t reduce128_6q(U128 x, uint64_t q, uint64_t r64, uint64_t r64p, uint64_t inv1) {
  const uint64_t a = mul_shoup_lazy(x.hi, r64, r64p, q);  // [0, 4q)
  const uint64_t b = x.lo - mulhi64(x.lo, inv1) * q;      // [0, 2q)
  return a + b;                                            // [0, 6q) < 2^63
}

// x mod q for x.hi < 2^64.
__device__ __forceinline__ uint64_t reduce128_lazy(U128 x, uint64_t q, uint64_t r64, uint64_t r64p, uint64_t inv1) {
  uint64_t s = reduce128_6q(x, q, r64, r64p, inv1);
  s = s >= 4 * q ? s - 4 * q : s;
  s = s >= 2 * q ? s - 2 * q : s;
  return s >= q ? s - q : s;
}


__device__ __forceinline__ uint64_t acc3_reduce(const Acc3& A, const uint64_t q, uint64_t r64, uint64_t r64p,
                                                uint64_t inv1) {
  return reduce128_lazy(acc3_value(A), q, r64, r64p, inv1);
}
// The same sum, congruent mod q, in [0, 6q).
__device__ __forceinline__ uint64_t acc3_reduce_6q(const Acc3& A, const uint64_t q, uint64_t r64, uint64_t r64p,
                                                   uint64_t inv1) {
  return reduce128_6q(acc3_value(A), q, r64, r64p, inv1);
}

__device__ __forceinline__ uint64_t add_mod(uint64_t a, uint64_t b, uint64_t q) {
  uint64_t s = a + b;
  return s >= q ? s - q : s;
}
__device__ __forceinline__ uint64_t sub_mod(uint64_t a, uint64_t b, uint64_t q) { return a >= b ? a - b : a + q - b; }

// Full product a*b mod q of two reduced values.
__device__ __forceinline__ uint64_t mul_mod(uint64_t a, uint64_t b, uint64_t q, uint64_t r64, uint64_t r64p,
                                            uint64_t inv1) {
  return reduce128(mul_wide(a, b), q, r64, r64p, inv1);
}

// Exact dot products in two operand forms, chosen per parameter set: NARROW
// (every operand below 2^60: 30-bit halves and Acc3 column sums) and WIDE
// (operands below 2^62: full 64x64 -> 128-bit products; 8 of them sum below
// 2^127, within reduce128's range).  Either form takes 8 products between
// reductions.  Tables of constants store them as lo30 | hi30 << 32 (hi30 up
// to 32 bits for constants below 2^62).
struct SplitN {
  uint32_t l, h;
};
struct SplitWd {
  uint64_t v;
};
template <bool WIDE>
using Split = typename std::conditional<WIDE, SplitWd, SplitN>::type;
template <bool WIDE>
using AccT = typename std::conditional<WIDE, U128, Acc3>::type;

template <bool WIDE>
__device__ __forceinline__ Split<WIDE> split_word(uint64_t v) {
  if constexpr (WIDE) return SplitWd{v};
  else return SplitN{lo30(v), hi30(v)};
}
template <bool WIDE>
__device__ __forceinline__ Split<WIDE> split_table(uint64_t cw) {
  if constexpr (WIDE) return SplitWd{(cw & 0x3fffffffull) | ((cw >> 32) << 30)};
  else return SplitN{(uint32_t)cw, (uint32_t)(cw >> 32)};
}
template <bool WIDE>
__device__ __forceinline__ void acc_mac(AccT<WIDE>& A, const Split<WIDE>& x, const Split<WIDE>& c) {
  if constexpr (WIDE) mac(A, x.v, c.v);
  else acc3_mac(A, x.l, x.h, c.l, c.h);
}
// the sum mod q, in [0, q)
template <bool WIDE>
__device__ __forceinline__ uint64_t acc_reduce(const AccT<WIDE>& A, uint64_t q, uint64_t r64, uint64_t r64p,
                                               uint64_t inv1) {
  if constexpr (WIDE) return reduce128(A, q, r64, r64p, inv1);
  else return acc3_reduce(A, q, r64, r64p, inv1);
}
// the sum mod q, in [0, 6q) (NARROW) or [0, q) (WIDE)
template <bool WIDE>
__device__ __forceinline__ uint64_t acc_reduce_6q(const AccT<WIDE>& A, uint64_t q, uint64_t r64, uint64_t r64p,
                                                  uint64_t inv1) {
  if constexpr (WIDE) return reduce128(A, q, r64, r64p, inv1);
  else return acc3_reduce_6q(A, q, r64, r64p, inv1);
}

}  // namespace ckks
