// Host-side integer helpers for parameter set-up: modular arithmetic on
// 64-bit moduli, primality, roots of unity and the precomputed constants the
// kernels consume.  Nothing here runs per coefficient; it builds tables once
// per context.
#pragma once
#include <stdint.h>

namespace ckks {
namespace host {

typedef unsigned __int128 u128;

inline uint64_t mulmod(uint64_t a, uint64_t b, uint64_t m) { return (uint64_t)((u128)a * b % m); }

inline uint64_t powmod(uint64_t a, uint64_t e, uint64_t m) {
  uint64_t r = 1 % m;
  a %= m;
  for (; e; e >>= 1) {
    if (e & 1) r = mulmod(r, a, m);
    a = mulmod(a, a, m);
  }
  return r;
}

// Inverse modulo a prime (Fermat).
inline uint64_t invmod(uint64_t a, uint64_t m) { return powmod(a % m, m - 2, m); }

// Shoup quotient floor(w * 2^64 / m) for w < m.
inline uint64_t shoup(uint64_t w, uint64_t m) { return (uint64_t)(((u128)w << 64) / m); }

// Strong-probable-prime test to one base.
inline bool sprp(uint64_t n, uint64_t a) {
  uint64_t d = n - 1;
  int s = 0;
  while (!(d & 1)) {
    d >>= 1;
    ++s;
  }
  uint64_t x = powmod(a, d, n);
  if (x == 1 || x == n - 1) return true;
  for (int i = 1; i < s; ++i) {
    x = mulmod(x, x, n);
    if (x == n - 1) return true;
  }
  return false;
}

// Deterministic for all 64-bit n: the first twelve primes as bases suffice
// below 3.3e24 (Sorenson and Webster).
inline bool is_prime(uint64_t n) {
  static const uint64_t small[12] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
  if (n < 2) return false;
  for (uint64_t p : small) {
    if (n == p) return true;
    if (n % p == 0) return false;
  }
  for (uint64_t p : small)
    if (!sprp(n, p)) return false;
  return true;
}

inline uint32_t bit_reverse(uint32_t x, int bits) {
  uint32_t r = 0;
  for (int i = 0; i < bits; ++i) {
    r = (r << 1) | (x & 1);
    x >>= 1;
  }
  return r;
}

// Smallest primitive 2N-th root of unity modulo prime m (m = 1 mod 2N);
// 0 if there is none.
inline uint64_t smallest_primitive_root_2n(uint64_t m, int log_n) {
  uint64_t n = 1ull << log_n, two_n = 2 * n;
  if ((m - 1) % two_n) return 0;
  uint64_t r = 0;
  for (uint64_t x = 2; x < m && !r; ++x) {
    uint64_t c = powmod(x, (m - 1) / two_n, m);
    if (powmod(c, n, m) == m - 1) r = c;
  }
  if (!r) return 0;
  uint64_t step = mulmod(r, r, m), cur = r, best = r;
  for (uint64_t k = 0; k < n; ++k) {  // odd powers r^(2k+1)
    if (cur < best) best = cur;
    cur = mulmod(cur, step, m);
  }
  return best;
}

}  // namespace host
}  // namespace ckks
