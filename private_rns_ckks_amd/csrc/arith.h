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
//   U128 / mac     exact 128-bit accumulation of 64x64 products and one
//                  Barrett-style reduction per output.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ uint64_t reduce_2q(uint64_t a, uint64_t q) { return a >= q ? a - q : a; }

// a mod q for any 64-bit a, given inv1 = floor(2^64 / q).
__device__ __forceinline__ uint64_t reduce64(uint64_t a, uint64_t q, uint64_t inv1) {
  uint64_t r = a - mulhi64(a, inv1) * q;  // Shoup with w = 1: r in [0, 2q)
  return reduce_2q(r, q);
}

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

}  // namespace ckks
