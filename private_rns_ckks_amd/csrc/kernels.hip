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
#include "convert.h"
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

// ModUp for digit blockIdx.y of batch item blockIdx.z.
// x: the digit limbs already multiplied by [qhat_i^-1]_{q_i} (canonical y_i),
// [level+1][N] per item.  out: [beta][next][N] per item; for every target limb
// t outside the digit, out_t = sum_i y_i [qhat_i]_{m_t} mod m_t (exact,
// left in the range conv_dot_c gives).
// Constants [qhat_i]_{m_t}: [NS][next], split into 30-bit halves, zero rows
// past the digit's size.  WIDE: some prime is at least 2^60 (full-width
// products).  Every thread converts two adjacent coefficients (16-byte loads
// and stores), so each target's constants serve two words; limbs are
// addressed as a wave-uniform base plus a 32-bit lane offset.
template <int NS, bool WIDE>
__global__ __launch_bounds__(256) void modup_kernel(ModUpArgs a) {
  const int j = blockIdx.y;
  const int lo = a.lo[j], hi = a.hi[j], na = hi - lo;
  const ConstU64 conv = (ConstU64)(a.tables + a.offset[j] + 2 * na);
  const ConstPrime prime = (ConstPrime)a.prime;
  const uint32_t c2 = blockIdx.x * blockDim.x + threadIdx.x;  // coefficients 2*c2, 2*c2+1
  const uint64_t* x = a.x + blockIdx.z * a.x_bstride + (uint64_t)lo * a.n;
  uint64_t* out = a.out + blockIdx.z * a.out_bstride + (uint64_t)j * a.next * a.n;
  Split<WIDE> y0[NS], y1[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ulonglong2 v = make_ulonglong2(0, 0);
    if (i < na) v = nttc::at_u32(reinterpret_cast<const ulonglong2*>(x + (uint64_t)i * a.n), c2);
    y0[i] = split_word<WIDE>(v.x);
    y1[i] = split_word<WIDE>(v.y);
  }
  for (int t = 0; t < a.next; ++t) {
    if (t >= lo && t < hi) continue;
    const RedConst pc = red_const(prime, t <= a.level ? t : a.L + (t - a.level - 1));
    uint64_t cw[NS];
    conv_consts<NS>(conv + t, a.next, cw);
    const uint64_t r0 = conv_dot_c<NS, WIDE>(y0, cw, pc);
    const uint64_t r1 = conv_dot_c<NS, WIDE>(y1, cw, pc);
    nttc::at_u32(reinterpret_cast<ulonglong2*>(out + (uint64_t)t * a.n), c2) = make_ulonglong2(r0, r1);
  }
}

// ModDown conversion for component blockIdx.y of item blockIdx.z.
// The special limbs of acc hold y_k = z_k [phat_k^-1]_{p_k} (canonical,
// coefficient form).  Centred lift: y_k counts as negative when
// y_k > (p_k-1)/2, and then sum_k ybar_k [phat_k P^-1]_{q_i} =
// sum_k y_k [1/p_k]_{q_i} - #negative  (mod q_i).  w: [2][level+1][N] per item,
// in the range conv_dot_c gives.
// Constants [1/p_k]_{q_i}: [NS][L], split into 30-bit halves, zero rows past K.
// Two adjacent coefficients per thread, as ModUp.
template <int NS, bool WIDE>
__global__ __launch_bounds__(256) void moddown_conv_kernel(ModDownArgs a) {
  const int nq = a.level + 1;
  const ConstU64 conv = (ConstU64)a.conv;
  const ConstPrime prime = (ConstPrime)a.prime;
  const uint32_t c2 = blockIdx.x * blockDim.x + threadIdx.x;  // coefficients 2*c2, 2*c2+1
  const int comp = blockIdx.y;
  const uint64_t* acc = a.acc + blockIdx.z * a.acc_bstride + (uint64_t)(comp * a.acc_comp_limbs + a.acc_k0) * a.n;
  Split<WIDE> y0[NS], y1[NS];
  uint32_t neg0 = 0, neg1 = 0;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    ulonglong2 v = make_ulonglong2(0, 0);
    if (k < a.K) {
      v = nttc::at_u32(reinterpret_cast<const ulonglong2*>(acc + (uint64_t)k * a.n), c2);
      const uint64_t half = prime[a.L + k].q >> 1;
      neg0 += v.x > half ? 1u : 0u;
      neg1 += v.y > half ? 1u : 0u;
    }
    y0[k] = split_word<WIDE>(v.x);
    y1[k] = split_word<WIDE>(v.y);
  }
  uint64_t* w = a.w + blockIdx.z * a.w_bstride + (uint64_t)comp * nq * a.n;
  for (int i = 0; i < nq; ++i) {
    const RedConst pc = red_const(prime, i);
    uint64_t cw[NS];
    conv_consts<NS>(conv + i, a.L, cw);
    const uint64_t r0 = sub_mod(conv_dot_c<NS, WIDE>(y0, cw, pc), neg0, pc.q);
    const uint64_t r1 = sub_mod(conv_dot_c<NS, WIDE>(y1, cw, pc), neg1, pc.q);
    nttc::at_u32(reinterpret_cast<ulonglong2*>(w + (uint64_t)i * a.n), c2) = make_ulonglong2(r0, r1);
  }
}

// d0 = a0 b0, d1 = a0 b1 + a1 b0, d2 = a1 b1 on limb blockIdx.y.
template <bool WIDE>
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
  const Split<WIDE> sa0 = split_word<WIDE>(a0), sa1 = split_word<WIDE>(a1);
  const Split<WIDE> sb0 = split_word<WIDE>(b0), sb1 = split_word<WIDE>(b1);
  AccT<WIDE> m0{}, m1{}, m2{};
  acc_mac<WIDE>(m0, sa0, sb0);
  acc_mac<WIDE>(m1, sa0, sb1);
  acc_mac<WIDE>(m1, sa1, sb0);
  acc_mac<WIDE>(m2, sa1, sb1);
  d[off] = acc_reduce<WIDE>(m0, pc.q, pc.r64, pc.r64p, pc.inv1);
  d[lim + off] = acc_reduce<WIDE>(m1, pc.q, pc.r64, pc.r64p, pc.inv1);
  d[2 * lim + off] = acc_reduce<WIDE>(m2, pc.q, pc.r64, pc.r64p, pc.inv1);
}

// BSGS inner sums: inner[o][g][comp][i] = sum_c sum_b diag[o][c][g][b][i] * baby[b][c][comp][i].
// A workgroup owns 256 coefficients of limb i for output o and loops over the
// giant steps g; the (c, b) terms go in groups of 8 (the split accumulator's
// capacity) with every load of a group issued before its products.  The
// diagonals stream from HBM once; the baby-step words a thread needs are the
// same for every g and every o, and the workgroup order below keeps the
// workgroups of one coefficient tile (all o) together on one XCD, so they are
// served by that XCD's L2.
template <bool WIDE>
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
      AccT<WIDE> s0{}, s1{};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const Split<WIDE> p = split_word<WIDE>(pt[k]);
        acc_mac<WIDE>(s0, p, split_word<WIDE>(c0[k]));
        acc_mac<WIDE>(s1, p, split_word<WIDE>(c1[k]));
      }
      r0 = add_mod(r0, acc_reduce<WIDE>(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r1 = add_mod(r1, acc_reduce<WIDE>(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
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
template <bool WIDE>
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
      AccT<WIDE> s0{}, s1{}, s1b{}, s2{};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const Split<WIDE> da = split_word<WIDE>(d0[k]), db = split_word<WIDE>(d1[k]);
        const Split<WIDE> xu = split_word<WIDE>(x0[k]), xv = split_word<WIDE>(x1[k]);
        acc_mac<WIDE>(s0, da, xu);
        acc_mac<WIDE>(s1, da, xv);
        acc_mac<WIDE>(s1b, db, xu);
        acc_mac<WIDE>(s2, db, xv);
      }
      r0 = add_mod(r0, acc_reduce<WIDE>(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r1 = add_mod(r1, acc_reduce<WIDE>(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r1 = add_mod(r1, acc_reduce<WIDE>(s1b, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
      r2 = add_mod(r2, acc_reduce<WIDE>(s2, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
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
template <int MAXG, bool WIDE>
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
    Split<WIDE> sc0[8], sc1[8];
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
      sc0[k] = split_word<WIDE>(x0);
      sc1[k] = split_word<WIDE>(x1);
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
        AccT<WIDE> s0{}, s1{};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const Split<WIDE> p = split_word<WIDE>(pt[k]);
          acc_mac<WIDE>(s0, p, sc0[k]);
          acc_mac<WIDE>(s1, p, sc1[k]);
        }
        r0[g] = add_mod(r0[g], acc_reduce<WIDE>(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1[g] = add_mod(r1[g], acc_reduce<WIDE>(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
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
template <int MAXG, bool WIDE>
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
    Split<WIDE> xu[8], xv[8];
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
      xu[k] = split_word<WIDE>(x0);
      xv[k] = split_word<WIDE>(x1);
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
        AccT<WIDE> s0{}, s1{}, s1b{}, s2{};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const Split<WIDE> da = split_word<WIDE>(d0[k]), db = split_word<WIDE>(d1[k]);
          acc_mac<WIDE>(s0, da, xu[k]);
          acc_mac<WIDE>(s1, da, xv[k]);
          acc_mac<WIDE>(s1b, db, xu[k]);
          acc_mac<WIDE>(s2, db, xv[k]);
        }
        r0[g] = add_mod(r0[g], acc_reduce<WIDE>(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1[g] = add_mod(r1[g], acc_reduce<WIDE>(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1[g] = add_mod(r1[g], acc_reduce<WIDE>(s1b, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r2[g] = add_mod(r2[g], acc_reduce<WIDE>(s2, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
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

// out = sum_t K_t x_t mod q_i.  Products of reduced words (< q^2 < 2^124)
// are summed in 128 bits, eight at a time (below 2^127, as reduce128 needs),
// and the partial sums added mod q.
__global__ void term_mac_kernel(TermMacArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int comp = blockIdx.y / a.nl, i = blockIdx.y % a.nl;
  const PrimeConst pc = a.prime[i];
  const uint64_t off = blockIdx.z * a.x_bstride + comp * a.x_comp + ((uint64_t)i << a.log_n) + c;
  uint64_t r = 0;
  for (int t0 = 0; t0 < a.nt; t0 += 8) {
    U128 s = {0, 0};
    const int t1 = min(a.nt, t0 + 8);
    for (int t = t0; t < t1; ++t) {
      const int64_t kt = a.k[t];
      uint64_t k = reduce64(kt < 0 ? (uint64_t)(-kt) : (uint64_t)kt, pc.q, pc.inv1);
      if (kt < 0 && k) k = pc.q - k;
      mac(s, k, a.x[t][off]);
    }
    r = add_mod(r, reduce128(s, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
  }
  if (a.has_add && comp == 0) r = add_mod(r, a.add0[i], pc.q);
  a.out[blockIdx.z * a.out_bstride + ((uint64_t)blockIdx.y << a.log_n) + c] = r;
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
  auto fn = conv_rows(c->alpha) == 8 ? (c->wide ? modup_kernel<8, true> : modup_kernel<8, false>)
                                     : (c->wide ? modup_kernel<16, true> : modup_kernel<16, false>);
  hipLaunchKernelGGL(fn, dim3(c->N / 512, beta, batch), dim3(256), 0, s, a);  // two coefficients per thread
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_moddown_conv(Ctx* c, hipStream_t s, ModDownArgs& a, int batch) {
  TraceScope ts(c, s, "moddown_conv", (double)batch * 2 * (a.K + (double)(a.level + 1) * (a.K + 1)) * c->N);
  auto fn = conv_rows(c->K) == 8 ? (c->wide ? moddown_conv_kernel<8, true> : moddown_conv_kernel<8, false>)
                                 : (c->wide ? moddown_conv_kernel<16, true> : moddown_conv_kernel<16, false>);
  hipLaunchKernelGGL(fn, dim3(c->N / 512, 2, batch), dim3(256), 0, s, a);  // two coefficients per thread
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_tensor(Ctx* c, hipStream_t s, TensorArgs& a, int batch) {
  TraceScope ts(c, s, "tensor", (double)batch * (a.level + 1) * 7 * c->N);
  hipLaunchKernelGGL(c->wide ? tensor_kernel<true> : tensor_kernel<false>, dim3(c->N / 256, a.level + 1, batch),
                     dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_ptmac(Ctx* c, hipStream_t s, PtMacArgs& a, int n_out) {
  TraceScope ts(c, s, "ptmac", (double)n_out * a.n2 * (a.level + 1) * 2 * (a.n_in * a.n1 + 1) * c->N);
  auto fn = a.n2 <= 8 ? (c->wide ? ptmac_regs_kernel<8, true> : ptmac_regs_kernel<8, false>)
                      : (c->wide ? ptmac_kernel<true> : ptmac_kernel<false>);
  hipLaunchKernelGGL(fn, dim3(n_out, a.level + 1, c->N / 256), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_ctmac(Ctx* c, hipStream_t s, CtMacArgs& a, int n_out) {
  TraceScope ts(c, s, "ctmac", (double)n_out * a.n2 * (a.level + 1) * (4 * a.n_in * a.n1 + 3) * c->N);
  auto fn = a.n2 <= 8 ? (c->wide ? ctmac_regs_kernel<8, true> : ctmac_regs_kernel<8, false>)
                      : (c->wide ? ctmac_kernel<true> : ctmac_kernel<false>);
  hipLaunchKernelGGL(fn, dim3(n_out, a.level + 1, c->N / 256), dim3(256), 0, s, a);
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

int launch_term_mac(Ctx* c, hipStream_t s, TermMacArgs& a, int batch) {
  if (a.nt < 0 || a.nt > kMaxTerms || a.nl < 1 || a.nl > 64) return set_error(CKKS_EINTERNAL, "bad term count");
  TraceScope ts(c, s, "term_mac", (double)batch * 2 * a.nl * (a.nt + (a.nt + 7) / 8) * c->N);
  hipLaunchKernelGGL(term_mac_kernel, dim3(c->N / 256, 2 * a.nl, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

}  // namespace ckks
