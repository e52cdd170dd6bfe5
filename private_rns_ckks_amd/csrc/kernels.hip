// Non-NTT kernels of the hot path: Galois automorphism, ModUp and ModDown
// basis conversion, the key-switch inner product, the final combination
// steps, rescale, ciphertext tensor product and the plaintext MAC.
//
// All kernels are elementwise over the N coefficients of a limb: one thread
// per coefficient, blockIdx.x over coefficient tiles of 256, blockIdx.y over
// limbs (or digits / components), blockIdx.z over batch items.  Limb-major
// layout makes every load and store a contiguous 64-bit access per lane.
#include "arith.h"
#include "automorph.h"
#include "kernels.h"
#include "ntt_core.h"

namespace ckks {

namespace {

__global__ void automorph_ntt_kernel(const uint64_t* in, uint64_t* out, uint64_t pstride, uint32_t g, int log_n) {
  const uint32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t base = blockIdx.z * pstride + ((uint64_t)blockIdx.y << log_n);
  out[base + j] = in[base + automorph_src(j, g, log_n)];
}

// Coefficient form: output coefficient r takes input coefficient u = r/g mod 2N,
// negated when u >= N (X^N = -1).
__global__ void automorph_coeff_kernel(const uint64_t* in, uint64_t* out, uint64_t pstride, uint32_t ginv, int log_n,
                                       const PrimeConst* pc) {
  const uint32_t r = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t n = 1u << log_n;
  const uint64_t base = blockIdx.z * pstride + ((uint64_t)blockIdx.y << log_n);
  const uint32_t u = (r * ginv) & (2 * n - 1);
  const uint64_t q = pc[blockIdx.y].q;
  if (u < n) {
    out[base + r] = in[base + u];
  } else {
    const uint64_t v = in[base + u - n];
    out[base + r] = v ? q - v : 0;
  }
}

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

// Split multiply-accumulate of NS sources against one target's constants
// (rows of a zero-padded table, stride `stride`), reduced mod the target q:
// in [0, 6q) for NS = 8, in [0, q) for NS = 16.  Both ranges are valid inputs
// of the forward NTT that follows (lazy butterflies start from words below
// 6q and stay below 70q < 2^64 for q < 2^57; the others accept words below
// 8q).  NS is 8 or 16; sources past the real count have zero constants and
// words.
template <int NS>
__device__ __forceinline__ uint64_t conv_dot(const uint32_t (&yl)[NS], const uint32_t (&yh)[NS], ConstU64 conv,
                                             int stride, const RedConst& pc) {
  uint64_t cw[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) cw[i] = conv[i * stride];
  uint64_t r = 0;
#pragma unroll
  for (int g = 0; g < NS; g += 8) {
    Acc3 A = {0, 0, 0};
#pragma unroll
    for (int i = g; i < g + 8; ++i) acc3_mac(A, yl[i], yh[i], (uint32_t)cw[i], (uint32_t)(cw[i] >> 32));
    if (NS == 8) return acc3_reduce_6q(A, pc.q, pc.r64, pc.r64p, pc.inv1);
    const uint64_t v = acc3_reduce(A, pc.q, pc.r64, pc.r64p, pc.inv1);
    r = g ? add_mod(r, v, pc.q) : v;
  }
  return r;
}

// ModUp for digit blockIdx.y of batch item blockIdx.z.
// x: the digit limbs already multiplied by [qhat_i^-1]_{q_i} (canonical y_i),
// [level+1][N] per item.  out: [beta][next][N] per item; for every target limb
// t outside the digit, out_t = sum_i y_i [qhat_i]_{m_t} mod m_t (exact,
// left in the range conv_dot gives).
// Constants [qhat_i]_{m_t}: [NS][next], split into 30-bit halves, zero rows
// past the digit's size.
template <int NS>
__global__ __launch_bounds__(256) void modup_kernel(ModUpArgs a) {
  const int j = blockIdx.y;
  const int lo = a.lo[j], hi = a.hi[j], na = hi - lo;
  const ConstU64 conv = (ConstU64)(a.tables + a.offset[j] + 2 * na);
  const ConstPrime prime = (ConstPrime)a.prime;
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t* x = a.x + blockIdx.z * a.x_bstride + (uint64_t)lo * a.n + c;
  uint64_t* out = a.out + blockIdx.z * a.out_bstride + (uint64_t)j * a.next * a.n + c;
  uint32_t yl[NS], yh[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const uint64_t y = i < na ? x[(uint64_t)i * a.n] : 0;
    yl[i] = lo30(y);
    yh[i] = hi30(y);
  }
  for (int t = 0; t < a.next; ++t) {
    if (t >= lo && t < hi) continue;
    const RedConst pc = red_const(prime, t <= a.level ? t : a.L + (t - a.level - 1));
    out[(uint64_t)t * a.n] = conv_dot<NS>(yl, yh, conv + t, a.next, pc);
  }
}

// ModDown conversion for component blockIdx.y of item blockIdx.z.
// The special limbs of acc hold y_k = z_k [phat_k^-1]_{p_k} (canonical,
// coefficient form).  Centred lift: y_k counts as negative when
// y_k > (p_k-1)/2, and then sum_k ybar_k [phat_k P^-1]_{q_i} =
// sum_k y_k [1/p_k]_{q_i} - #negative  (mod q_i).  w: [2][level+1][N] per item,
// in the range conv_dot gives.
// Constants [1/p_k]_{q_i}: [NS][L], split into 30-bit halves, zero rows past K.
template <int NS>
__global__ __launch_bounds__(256) void moddown_conv_kernel(ModDownArgs a) {
  const int nq = a.level + 1;
  const ConstU64 conv = (ConstU64)a.conv;
  const ConstPrime prime = (ConstPrime)a.prime;
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int comp = blockIdx.y;
  const uint64_t* acc = a.acc + blockIdx.z * a.acc_bstride + (uint64_t)(comp * a.next + nq) * a.n + c;
  uint32_t yl[NS], yh[NS];
  uint32_t neg = 0;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    uint64_t v = 0;
    if (k < a.K) {
      v = acc[(uint64_t)k * a.n];
      neg += v > (prime[a.L + k].q >> 1) ? 1u : 0u;
    }
    yl[k] = lo30(v);
    yh[k] = hi30(v);
  }
  uint64_t* w = a.w + blockIdx.z * a.w_bstride + (uint64_t)comp * nq * a.n + c;
  for (int i = 0; i < nq; ++i) {
    const RedConst pc = red_const(prime, i);
    w[(uint64_t)i * a.n] = sub_mod(conv_dot<NS>(yl, yh, conv + i, a.L, pc), neg, pc.q);
  }
}

// d0 = a0 b0, d1 = a0 b1 + a1 b0, d2 = a1 b1 on limb blockIdx.y.
__global__ __launch_bounds__(256) void tensor_kernel(TensorArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y;
  const PrimeConst pc = a.prime[i];
  const uint64_t lim = (uint64_t)(a.level + 1) * a.n;
  const uint64_t off = (uint64_t)i * a.n + c;
  const uint64_t* x = a.a + blockIdx.z * a.in_bstride;
  const uint64_t* y = a.b + blockIdx.z * a.b_bstride;
  uint64_t* d = a.out + blockIdx.z * a.out_bstride;
  const uint64_t a0 = x[off], a1 = x[lim + off], b0 = y[off], b1 = y[a.b_comp + off];
  const uint32_t a0l = lo30(a0), a0h = hi30(a0), a1l = lo30(a1), a1h = hi30(a1);
  const uint32_t b0l = lo30(b0), b0h = hi30(b0), b1l = lo30(b1), b1h = hi30(b1);
  Acc3 m0 = {0, 0, 0}, m1 = {0, 0, 0}, m2 = {0, 0, 0};
  acc3_mac(m0, a0l, a0h, b0l, b0h);
  acc3_mac(m1, a0l, a0h, b1l, b1h);
  acc3_mac(m1, a1l, a1h, b0l, b0h);
  acc3_mac(m2, a1l, a1h, b1l, b1h);
  d[off] = acc3_reduce(m0, pc.q, pc.r64, pc.r64p, pc.inv1);
  d[lim + off] = acc3_reduce(m1, pc.q, pc.r64, pc.r64p, pc.inv1);
  d[2 * lim + off] = acc3_reduce(m2, pc.q, pc.r64, pc.r64p, pc.inv1);
}

// BSGS inner sums: inner[o][g][comp][i] = sum_c sum_b diag[o][c][g][b][i] * baby[b][c][comp][i].
// A workgroup owns 256 coefficients of limb i for output o and loops over the
// giant steps g; the (c, b) terms go in groups of 8 (the split accumulator's
// capacity) with every load of a group issued before its products.  The
// diagonals stream from HBM once; the baby-step words a thread needs are the
// same for every g and every o, and the workgroup order below keeps the
// workgroups of one coefficient tile (all o) together on one XCD, so they are
// served by that XCD's L2.
__global__ __launch_bounds__(256) void ptmac_kernel(PtMacArgs a) {
  const nttc::GridPos gp = nttc::row_grid_pos();  // grid (n_out, limbs, N/256): o fastest
  const int o = (int)gp.tile, i = gp.job;
  const uint32_t c = (uint32_t)gp.item * blockDim.x + threadIdx.x;
  const RedConst pc = red_const((ConstPrime)a.prime, i);
  const uint64_t limbs = (uint64_t)(a.level + 1);
  const uint64_t off = (uint64_t)i * a.n + c;
  const uint64_t ln = limbs * a.n;
  const int terms = a.n_in * a.n1;
  for (int g = 0; g < a.n2; ++g) {
    uint64_t r0 = 0, r1 = 0;
    for (int t0 = 0; t0 < terms; t0 += 8) {
      uint64_t pt[8], c0[8], c1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        pt[k] = c0[k] = c1[k] = 0;
        const int t = t0 + k;
        if (t < terms) {
          const int ci = t / a.n1, b = t % a.n1;
          pt[k] = a.diags[((((uint64_t)o * a.n_in + ci) * a.n2 + g) * a.n1 + b) * ln + off];
          const uint64_t* ct = a.baby + ((uint64_t)b * a.n_in + ci) * 2 * ln + off;
          c0[k] = ct[0];
          c1[k] = ct[ln];
        }
      }
      Acc3 s0 = {0, 0, 0}, s1 = {0, 0, 0};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t pl = lo30(pt[k]), ph = hi30(pt[k]);
        acc3_mac(s0, pl, ph, lo30(c0[k]), hi30(c0[k]));
        acc3_mac(s1, pl, ph, lo30(c1[k]), hi30(c1[k]));
      }
      r0 = add_mod(r0, acc3_reduce(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r1 = add_mod(r1, acc3_reduce(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
    }
    uint64_t* out = a.out + ((uint64_t)o * a.n2 + g) * 2 * ln;
    out[off] = r0;
    out[ln + off] = r1;
  }
}

// Encrypted-weight BSGS inner sums, before relinearisation:
//   T[o][g] = sum_c sum_b tensor(diag[o][c][g][b], baby[b][c])
// with tensor(D, X) = (D0 X0, D0 X1 + D1 X0, D1 X1).  Same tiling and
// workgroup order as ptmac_kernel; four split accumulators per group of 8
// terms (the middle part keeps its two products apart, so no accumulator
// takes more than 8 products).
__global__ __launch_bounds__(256) void ctmac_kernel(CtMacArgs a) {
  const nttc::GridPos gp = nttc::row_grid_pos();  // grid (n_out, limbs, N/256): o fastest
  const int o = (int)gp.tile, i = gp.job;
  const uint32_t c = (uint32_t)gp.item * blockDim.x + threadIdx.x;
  const RedConst pc = red_const((ConstPrime)a.prime, i);
  const uint64_t limbs = (uint64_t)(a.level + 1);
  const uint64_t off = (uint64_t)i * a.n + c;
  const uint64_t ln = limbs * a.n;
  const int terms = a.n_in * a.n1;
  for (int g = 0; g < a.n2; ++g) {
    uint64_t r0 = 0, r1 = 0, r2 = 0;
    for (int t0 = 0; t0 < terms; t0 += 8) {
      uint64_t d0[8], d1[8], x0[8], x1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        d0[k] = d1[k] = x0[k] = x1[k] = 0;
        const int t = t0 + k;
        if (t < terms) {
          const int ci = t / a.n1, b = t % a.n1;
          const uint64_t* d = a.diags + ((((uint64_t)o * a.n_in + ci) * a.n2 + g) * a.n1 + b) * 2 * ln + off;
          const uint64_t* x = a.baby + ((uint64_t)b * a.n_in + ci) * 2 * ln + off;
          d0[k] = d[0];
          d1[k] = d[ln];
          x0[k] = x[0];
          x1[k] = x[ln];
        }
      }
      Acc3 s0 = {0, 0, 0}, s1 = {0, 0, 0}, s1b = {0, 0, 0}, s2 = {0, 0, 0};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t al = lo30(d0[k]), ah = hi30(d0[k]), bl = lo30(d1[k]), bh = hi30(d1[k]);
        const uint32_t ul = lo30(x0[k]), uh = hi30(x0[k]), vl = lo30(x1[k]), vh = hi30(x1[k]);
        acc3_mac(s0, al, ah, ul, uh);
        acc3_mac(s1, al, ah, vl, vh);
        acc3_mac(s1b, bl, bh, ul, uh);
        acc3_mac(s2, bl, bh, vl, vh);
      }
      r0 = add_mod(r0, acc3_reduce(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r1 = add_mod(r1, acc3_reduce(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r1 = add_mod(r1, acc3_reduce(s1b, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r2 = add_mod(r2, acc3_reduce(s2, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
    }
    uint64_t* out = a.out + ((uint64_t)o * a.n2 + g) * 3 * ln;
    out[off] = r0;
    out[ln + off] = r1;
    out[2 * ln + off] = r2;
  }
}

// The same sums with the loops swapped, for n2 <= MAXG: the baby-step words
// of a group of 8 (c, b) terms are loaded once and used for every giant step,
// whose running sums stay in registers; only the diagonals stream.
template <int MAXG>
__global__ __launch_bounds__(256) void ptmac_regs_kernel(PtMacArgs a) {
  const nttc::GridPos gp = nttc::row_grid_pos();  // grid (n_out, limbs, N/256): o fastest
  const int o = (int)gp.tile, i = gp.job;
  const uint32_t c = (uint32_t)gp.item * blockDim.x + threadIdx.x;
  const RedConst pc = red_const((ConstPrime)a.prime, i);
  const uint64_t limbs = (uint64_t)(a.level + 1);
  const uint64_t off = (uint64_t)i * a.n + c;
  const uint64_t ln = limbs * a.n;
  const int terms = a.n_in * a.n1;
  uint64_t r0[MAXG], r1[MAXG];
#pragma unroll
  for (int g = 0; g < MAXG; ++g) r0[g] = r1[g] = 0;
  for (int t0 = 0; t0 < terms; t0 += 8) {
    uint32_t c0l[8], c0h[8], c1l[8], c1h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = t0 + k;
      uint64_t x0 = 0, x1 = 0;
      if (t < terms) {
        const int ci = t / a.n1, b = t % a.n1;
        const uint64_t* ct = a.baby + ((uint64_t)b * a.n_in + ci) * 2 * ln + off;
        x0 = ct[0];
        x1 = ct[ln];
      }
      c0l[k] = lo30(x0);
      c0h[k] = hi30(x0);
      c1l[k] = lo30(x1);
      c1h[k] = hi30(x1);
    }
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      if (g < a.n2) {
        uint64_t pt[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int t = t0 + k;
          pt[k] = 0;
          if (t < terms) {
            const int ci = t / a.n1, b = t % a.n1;
            pt[k] = a.diags[((((uint64_t)o * a.n_in + ci) * a.n2 + g) * a.n1 + b) * ln + off];
          }
        }
        Acc3 s0 = {0, 0, 0}, s1 = {0, 0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t pl = lo30(pt[k]), ph = hi30(pt[k]);
          acc3_mac(s0, pl, ph, c0l[k], c0h[k]);
          acc3_mac(s1, pl, ph, c1l[k], c1h[k]);
        }
        r0[g] = add_mod(r0[g], acc3_reduce(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1[g] = add_mod(r1[g], acc3_reduce(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < MAXG; ++g) {
    if (g < a.n2) {
      uint64_t* out = a.out + ((uint64_t)o * a.n2 + g) * 2 * ln;
      out[off] = r0[g];
      out[ln + off] = r1[g];
    }
  }
}

// ctmac_kernel with the loops swapped as in ptmac_regs_kernel (n2 <= MAXG).
template <int MAXG>
__global__ __launch_bounds__(256) void ctmac_regs_kernel(CtMacArgs a) {
  const nttc::GridPos gp = nttc::row_grid_pos();  // grid (n_out, limbs, N/256): o fastest
  const int o = (int)gp.tile, i = gp.job;
  const uint32_t c = (uint32_t)gp.item * blockDim.x + threadIdx.x;
  const RedConst pc = red_const((ConstPrime)a.prime, i);
  const uint64_t limbs = (uint64_t)(a.level + 1);
  const uint64_t off = (uint64_t)i * a.n + c;
  const uint64_t ln = limbs * a.n;
  const int terms = a.n_in * a.n1;
  uint64_t r0[MAXG], r1[MAXG], r2[MAXG];
#pragma unroll
  for (int g = 0; g < MAXG; ++g) r0[g] = r1[g] = r2[g] = 0;
  for (int t0 = 0; t0 < terms; t0 += 8) {
    uint32_t ul[8], uh[8], vl[8], vh[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = t0 + k;
      uint64_t x0 = 0, x1 = 0;
      if (t < terms) {
        const int ci = t / a.n1, b = t % a.n1;
        const uint64_t* x = a.baby + ((uint64_t)b * a.n_in + ci) * 2 * ln + off;
        x0 = x[0];
        x1 = x[ln];
      }
      ul[k] = lo30(x0);
      uh[k] = hi30(x0);
      vl[k] = lo30(x1);
      vh[k] = hi30(x1);
    }
#pragma unroll
    for (int g = 0; g < MAXG; ++g) {
      if (g < a.n2) {
        uint64_t d0[8], d1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int t = t0 + k;
          d0[k] = d1[k] = 0;
          if (t < terms) {
            const int ci = t / a.n1, b = t % a.n1;
            const uint64_t* d = a.diags + ((((uint64_t)o * a.n_in + ci) * a.n2 + g) * a.n1 + b) * 2 * ln + off;
            d0[k] = d[0];
            d1[k] = d[ln];
          }
        }
        Acc3 s0 = {0, 0, 0}, s1 = {0, 0, 0}, s1b = {0, 0, 0}, s2 = {0, 0, 0};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t al = lo30(d0[k]), ah = hi30(d0[k]), bl = lo30(d1[k]), bh = hi30(d1[k]);
          acc3_mac(s0, al, ah, ul[k], uh[k]);
          acc3_mac(s1, al, ah, vl[k], vh[k]);
          acc3_mac(s1b, bl, bh, ul[k], uh[k]);
          acc3_mac(s2, bl, bh, vl[k], vh[k]);
        }
        r0[g] = add_mod(r0[g], acc3_reduce(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1[g] = add_mod(r1[g], acc3_reduce(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1[g] = add_mod(r1[g], acc3_reduce(s1b, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r2[g] = add_mod(r2[g], acc3_reduce(s2, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < MAXG; ++g) {
    if (g < a.n2) {
      uint64_t* out = a.out + ((uint64_t)o * a.n2 + g) * 3 * ln;
      out[off] = r0[g];
      out[ln + off] = r1[g];
      out[2 * ln + off] = r2[g];
    }
  }
}

__global__ void add_kernel(const uint64_t* x, const uint64_t* y, uint64_t* out, uint64_t bstride, int nl,
                           const PrimeConst* prime, int log_n) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y % nl;
  const uint64_t off = blockIdx.z * bstride + ((uint64_t)blockIdx.y << log_n) + c;
  out[off] = add_mod(x[off], y[off], prime[i].q);
}

// Every limb times a per-limb constant: out = in * k_i mod q_i (Shoup, with
// the constant's quotient), both components; in and out [2][nl][N] per item.
__global__ void const_mul_kernel(ConstMulArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y % a.nl;
  const uint64_t q = a.prime[i].q;
  const uint64_t off = ((uint64_t)blockIdx.y << a.log_n) + c;
  const uint64_t v = a.in[blockIdx.z * a.in_bstride + off];
  a.out[blockIdx.z * a.out_bstride + off] = reduce_4q(mul_shoup_lazy(v, a.k[i][0], a.k[i][1], q), q);
}

}  // namespace

#define LAUNCH_CHECK() CKKS_HIP_CHECK(hipGetLastError())

int launch_automorph_ntt(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t* out, int npoly, int nl, uint64_t pstride,
                         uint32_t g) {
  TraceScope ts(c, s, "automorph", 0);
  hipLaunchKernelGGL(automorph_ntt_kernel, dim3(c->N / 256, nl, npoly), dim3(256), 0, s, in, out, pstride, g,
                     (int)c->log_n);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_automorph_coeff(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t* out, int npoly, int nl,
                           uint64_t pstride, uint32_t ginv) {
  TraceScope ts(c, s, "automorph", 0);
  hipLaunchKernelGGL(automorph_coeff_kernel, dim3(c->N / 256, nl, npoly), dim3(256), 0, s, in, out, pstride, ginv,
                     (int)c->log_n, c->d_prime);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_modup(Ctx* c, hipStream_t s, ModUpArgs& a, int beta, int batch) {
  double units = 0;
  for (int j = 0; j < beta; ++j) {
    const int na = a.hi[j] - a.lo[j];
    units += na + (double)(a.next - na) * (na + 1);
  }
  TraceScope ts(c, s, "modup", units * batch * c->N);
  if (conv_rows(c->alpha) == 8)
    hipLaunchKernelGGL(modup_kernel<8>, dim3(c->N / 256, beta, batch), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(modup_kernel<16>, dim3(c->N / 256, beta, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_moddown_conv(Ctx* c, hipStream_t s, ModDownArgs& a, int batch) {
  TraceScope ts(c, s, "moddown_conv", (double)batch * 2 * (a.K + (double)(a.level + 1) * (a.K + 1)) * c->N);
  if (conv_rows(c->K) == 8)
    hipLaunchKernelGGL(moddown_conv_kernel<8>, dim3(c->N / 256, 2, batch), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(moddown_conv_kernel<16>, dim3(c->N / 256, 2, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_tensor(Ctx* c, hipStream_t s, TensorArgs& a, int batch) {
  TraceScope ts(c, s, "tensor", (double)batch * (a.level + 1) * 7 * c->N);
  hipLaunchKernelGGL(tensor_kernel, dim3(c->N / 256, a.level + 1, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_ptmac(Ctx* c, hipStream_t s, PtMacArgs& a, int n_out) {
  TraceScope ts(c, s, "ptmac", (double)n_out * a.n2 * (a.level + 1) * 2 * (a.n_in * a.n1 + 1) * c->N);
  if (a.n2 <= 8)
    hipLaunchKernelGGL(ptmac_regs_kernel<8>, dim3(n_out, a.level + 1, c->N / 256), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ptmac_kernel, dim3(n_out, a.level + 1, c->N / 256), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_ctmac(Ctx* c, hipStream_t s, CtMacArgs& a, int n_out) {
  TraceScope ts(c, s, "ctmac", (double)n_out * a.n2 * (a.level + 1) * (4 * a.n_in * a.n1 + 3) * c->N);
  if (a.n2 <= 8)
    hipLaunchKernelGGL(ctmac_regs_kernel<8>, dim3(n_out, a.level + 1, c->N / 256), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(ctmac_kernel, dim3(n_out, a.level + 1, c->N / 256), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_add(Ctx* c, hipStream_t s, const uint64_t* x, const uint64_t* y, uint64_t* out, int npoly, int nl,
               int ncomp, uint64_t bstride) {
  TraceScope ts(c, s, "add", 0);
  hipLaunchKernelGGL(add_kernel, dim3(c->N / 256, nl * ncomp, npoly), dim3(256), 0, s, x, y, out, bstride, nl,
                     c->d_prime, (int)c->log_n);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_const_mul(Ctx* c, hipStream_t s, ConstMulArgs& a, int batch) {
  TraceScope ts(c, s, "const_mul", (double)batch * 2 * a.nl * c->N);
  hipLaunchKernelGGL(const_mul_kernel, dim3(c->N / 256, 2 * a.nl, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

}  // namespace ckks
