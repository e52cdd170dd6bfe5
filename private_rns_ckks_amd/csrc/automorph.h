// Index map of the Galois automorphism X -> X^g in NTT form.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckks {

// Word j of an NTT-form limb holds a(psi^(2brv(j)+1)); after X -> X^g it must
// hold a(psi^(g(2brv(j)+1) mod 2N)), i.e. the input word returned here.
__device__ __forceinline__ uint32_t automorph_src(uint32_t j, uint32_t g, int log_n) {
  const uint32_t mask2n = (2u << log_n) - 1;
  const uint32_t e = 2 * (__brev(j) >> (32 - log_n)) + 1;
  const uint32_t eg = (e * g) & mask2n;
  return __brev((eg - 1) >> 1) >> (32 - log_n);
}

}  // namespace ckks
