// Basis-conversion helpers shared by the conversion kernels: constants read
// through the constant address space (wave-uniform indices become scalar
// loads into SGPRs) and the split multiply-accumulate of up to 16 sources
// against one target's constants.
#pragma once
#include "arith.h"
#include "internal.h"

namespace ckks {

// Read-only tables read with wave-uniform indices: through the constant
// address space the compiler fetches them with scalar loads, and the
// multiply-accumulates take them straight from SGPRs.
typedef const __attribute__((address_space(4))) uint64_t* ConstU64;
typedef const __attribute__((address_space(4))) PrimeConst* ConstPrime;

// The constants a reduction mod prime i needs.
struct RedConst {
  uint64_t q, r64, r64p, inv1;
};
__device__ __forceinline__ RedConst red_const(ConstPrime p, int i) {
  RedConst r;
  r.q = p[i].q;
  r.r64 = p[i].r64;
  r.r64p = p[i].r64p;
  r.inv1 = p[i].inv1;
  return r;
}

// Multiply-accumulate of NS sources against one target's constants (rows of
// a zero-padded table of split constants, stride `stride`), reduced mod the
// target q: NARROW, in [0, 6q) for NS = 8 and [0, q) for NS = 16; WIDE, in
// [0, q).  Both ranges are valid inputs of the forward NTT that follows (lazy
// butterflies start from words below 6q and stay below 70q < 2^64 for
// q < 2^57; Harvey butterflies accept words below 8q, strict ones below 4q).
// NS is 8 or 16; sources past the real count have zero constants and words.
// conv_consts reads one target's constants (scalar loads), conv_dot_c forms
// one coefficient's sum from them, so a thread converting several
// coefficients loads each constant once.
template <int NS>
__device__ __forceinline__ void conv_consts(ConstU64 conv, int stride, uint64_t (&cw)[NS]) {
#pragma unroll
  for (int i = 0; i < NS; ++i) cw[i] = conv[i * stride];
}

template <int NS, bool WIDE>
__device__ __forceinline__ uint64_t conv_dot_c(const Split<WIDE> (&y)[NS], const uint64_t (&cw)[NS],
                                               const RedConst& pc) {
  uint64_t r = 0;
#pragma unroll
  for (int g = 0; g < NS; g += 8) {
    AccT<WIDE> A{};
#pragma unroll
    for (int i = g; i < g + 8; ++i) acc_mac<WIDE>(A, y[i], split_table<WIDE>(cw[i]));
    if (NS == 8) return acc_reduce_6q<WIDE>(A, pc.q, pc.r64, pc.r64p, pc.inv1);
    const uint64_t v = acc_reduce<WIDE>(A, pc.q, pc.r64, pc.r64p, pc.inv1);
    r = g ? add_mod(r, v, pc.q) : v;
  }
  return r;
}

}  // namespace ckks
