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
// t outside the digit, out_t = sum_i y_i [qhat_i]_{m_t} mod m_t (exact).
// The conversion constants and target moduli are staged in LDS once per
// workgroup so the target loop reads them with broadcast LDS loads.
__global__ __launch_bounds__(256) void modup_kernel(ModUpArgs a) {
  __shared__ uint64_t s_conv[16 * kMaxExt];
  __shared__ uint64_t s_pc[4 * kMaxExt];
  const int j = blockIdx.y;
  const int lo = a.lo[j], hi = a.hi[j], na = hi - lo;
  const uint64_t* conv = a.tables + a.offset[j] + 2 * na;
  for (int k = threadIdx.x; k < na * a.next; k += blockDim.x) s_conv[k] = conv[k];
  for (int t = threadIdx.x; t < a.next; t += blockDim.x) {
    const PrimeConst& pc = a.prime[t <= a.level ? t : a.L + (t - a.level - 1)];
    s_pc[4 * t] = pc.q;
    s_pc[4 * t + 1] = pc.r64;
    s_pc[4 * t + 2] = pc.r64p;
    s_pc[4 * t + 3] = pc.inv1;
  }
  __syncthreads();
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const uint64_t* x = a.x + blockIdx.z * a.x_bstride + (uint64_t)lo * a.n + c;
  uint64_t* out = a.out + blockIdx.z * a.out_bstride + (uint64_t)j * a.next * a.n + c;
  uint32_t yl[16], yh[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < na) {
      const uint64_t y = x[(uint64_t)i * a.n];
      yl[i] = lo30(y);
      yh[i] = hi30(y);
    }
  }
  for (int t = 0; t < a.next; ++t) {
    if (t >= lo && t < hi) continue;
    const uint64_t q = s_pc[4 * t], r64 = s_pc[4 * t + 1], r64p = s_pc[4 * t + 2], inv1 = s_pc[4 * t + 3];
    Acc3 A = {0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < na) {
        const uint64_t cv = s_conv[i * a.next + t];
        acc3_mac(A, yl[i], yh[i], lo30(cv), hi30(cv));
      }
    }
    uint64_t r = acc3_reduce(A, q, r64, r64p, inv1);
    if (na > 8) {
      Acc3 B = {0, 0, 0};
#pragma unroll
      for (int i = 8; i < 16; ++i) {
        if (i < na) {
          const uint64_t cv = s_conv[i * a.next + t];
          acc3_mac(B, yl[i], yh[i], lo30(cv), hi30(cv));
        }
      }
      r = add_mod(r, acc3_reduce(B, q, r64, r64p, inv1), q);
    }
    out[(uint64_t)t * a.n] = r;
  }
}

// Inner product with the key digits for extended limb t = blockIdx.y:
// acc_b[t] = sum_j d_j[t] * evk_j.b[t], acc_a[t] likewise, where d_j[t] is the
// NTT-form input itself for limbs inside digit j and the NTT-form ModUp output
// otherwise.
__global__ __launch_bounds__(256) void inner_product_kernel(IPArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = blockIdx.y;
  const int item = blockIdx.z;
  const int keyl = t <= a.level ? t : a.L + (t - a.level - 1);
  const PrimeConst pc = a.prime[keyl];
  const uint64_t* evk = a.evk[item];
  const uint64_t LKN = (uint64_t)(a.L + a.K) * a.n;
  uint64_t rb = 0, ra = 0;
  // digits in groups of 8 (the split accumulator's capacity); within a group
  // every load is issued before the first multiply
  for (int j0 = 0; j0 < a.beta; j0 += 8) {
    uint64_t d[8], kb[8], ka[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj;
      if (j < a.beta) {
        const bool in_digit = t >= j * a.alpha && t < (j + 1) * a.alpha && t <= a.level;
        d[jj] = in_digit ? a.d[item * a.d_bstride + (uint64_t)t * a.n + c]
                         : a.ext[item * a.ext_bstride + ((uint64_t)j * a.next + t) * a.n + c];
        kb[jj] = evk[(2 * j) * LKN + (uint64_t)keyl * a.n + c];
        ka[jj] = evk[(2 * j + 1) * LKN + (uint64_t)keyl * a.n + c];
      }
    }
    Acc3 ab = {0, 0, 0}, aa = {0, 0, 0};
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < a.beta) {
        const uint32_t dl = lo30(d[jj]), dh = hi30(d[jj]);
        acc3_mac(ab, dl, dh, lo30(kb[jj]), hi30(kb[jj]));
        acc3_mac(aa, dl, dh, lo30(ka[jj]), hi30(ka[jj]));
      }
    }
    rb = add_mod(rb, acc3_reduce(ab, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
    ra = add_mod(ra, acc3_reduce(aa, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
  }
  uint64_t* out = a.acc + item * a.acc_bstride + (uint64_t)t * a.n + c;
  out[0] = rb;
  out[(uint64_t)a.next * a.n] = ra;
}

// ModDown conversion for component blockIdx.y of item blockIdx.z.
// The special limbs of acc hold y_k = z_k [phat_k^-1]_{p_k} (canonical,
// coefficient form).  Centred lift: y_k counts as negative when
// y_k > (p_k-1)/2, and then sum_k ybar_k [phat_k P^-1]_{q_i} =
// sum_k y_k [1/p_k]_{q_i} - #negative  (mod q_i).  w: [2][level+1][N] per item.
__global__ __launch_bounds__(256) void moddown_conv_kernel(ModDownArgs a) {
  __shared__ uint64_t s_conv[16 * 64];
  __shared__ uint64_t s_pc[4 * 64];
  const int nq = a.level + 1;
  for (int k = threadIdx.x; k < a.K * nq; k += blockDim.x) s_conv[k] = a.conv[(k / nq) * a.L + (k % nq)];
  for (int i = threadIdx.x; i < nq; i += blockDim.x) {
    const PrimeConst& pc = a.prime[i];
    s_pc[4 * i] = pc.q;
    s_pc[4 * i + 1] = pc.r64;
    s_pc[4 * i + 2] = pc.r64p;
    s_pc[4 * i + 3] = pc.inv1;
  }
  __syncthreads();
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int comp = blockIdx.y;
  const uint64_t* acc = a.acc + blockIdx.z * a.acc_bstride + (uint64_t)(comp * a.next + nq) * a.n + c;
  uint32_t yl[16], yh[16];
  uint32_t neg = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if (k < a.K) {
      const uint64_t v = acc[(uint64_t)k * a.n];
      neg += v > (a.prime[a.L + k].q >> 1) ? 1u : 0u;
      yl[k] = lo30(v);
      yh[k] = hi30(v);
    }
  }
  uint64_t* w = a.w + blockIdx.z * a.w_bstride + (uint64_t)comp * nq * a.n + c;
  for (int i = 0; i < nq; ++i) {
    const uint64_t q = s_pc[4 * i], r64 = s_pc[4 * i + 1], r64p = s_pc[4 * i + 2], inv1 = s_pc[4 * i + 3];
    Acc3 A = {0, 0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < a.K) {
        const uint64_t cv = s_conv[k * nq + i];
        acc3_mac(A, yl[k], yh[k], lo30(cv), hi30(cv));
      }
    }
    uint64_t r = acc3_reduce(A, q, r64, r64p, inv1);
    if (a.K > 8) {
      Acc3 B = {0, 0, 0};
#pragma unroll
      for (int k = 8; k < 16; ++k) {
        if (k < a.K) {
          const uint64_t cv = s_conv[k * nq + i];
          acc3_mac(B, yl[k], yh[k], lo30(cv), hi30(cv));
        }
      }
      r = add_mod(r, acc3_reduce(B, q, r64, r64p, inv1), q);
    }
    w[(uint64_t)i * a.n] = sub_mod(r, neg, q);
  }
}

// out[comp][i] = acc[comp][i] * P^-1 - w[comp][i]  (+ add[comp][i] gathered
// through X -> X^g when add_g != 0)  (+ accum[comp][i]).
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y;
  const int item = blockIdx.z;
  const PrimeConst pc = a.prime[i];
  const uint64_t q = pc.q;
  for (int comp = 0; comp < 2; ++comp) {
    const uint64_t av = a.acc[item * a.acc_bstride + ((uint64_t)comp * a.next + i) * a.n + c];
    const uint64_t wv = a.w[item * a.w_bstride + ((uint64_t)comp * (a.level + 1) + i) * a.n + c];
    uint64_t r = sub_mod(reduce_2q(mul_shoup(av, a.pinv[2 * i], a.pinv[2 * i + 1], q), q), wv, q);
    if (a.add[comp]) {
      const uint32_t g = a.add_g[item];
      const uint32_t src = g ? automorph_src(c, g, a.log_n) : c;
      r = add_mod(r, a.add[comp][item * a.add_bstride + (uint64_t)i * a.n + src], q);
    }
    if (a.accum) r = add_mod(r, a.accum[item * a.accum_bstride + ((uint64_t)comp * (a.level + 1) + i) * a.n + c], q);
    a.out[item * a.out_bstride + ((uint64_t)comp * a.out_comp_limbs + i) * a.n + c] = r;
  }
}

// Rescale, step 1: v = iNTT(c[l]) (canonical, 1/N applied) for both components;
// w_i = (vbar mod q_i) * [q_l^-1]_{q_i}, vbar the centered lift of v.
__global__ __launch_bounds__(256) void rescale_prep_kernel(RescaleArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int comp = blockIdx.y;
  const uint64_t v = a.v[blockIdx.z * a.v_bstride + (uint64_t)comp * a.n + c];
  const uint64_t ql = a.prime[a.level].q;
  const bool neg = v > (ql - 1) / 2;
  uint64_t* w = a.w + blockIdx.z * a.w_bstride + (uint64_t)comp * a.level * a.n + c;
  for (int i = 0; i < a.level; ++i) {
    const PrimeConst pc = a.prime[i];
    const uint64_t* rs = a.tab + ((uint64_t)a.level * a.L + i) * 4;
    uint64_t t = v >= pc.q ? reduce64(v, pc.q, pc.inv1) : v;
    if (neg) t = sub_mod(t, rs[2], pc.q);
    w[(uint64_t)i * a.n] = reduce_2q(mul_shoup(t, rs[0], rs[1], pc.q), pc.q);
  }
}

// Rescale, step 2: out_i = c_i * [q_l^-1]_{q_i} - NTT(w)_i.
__global__ __launch_bounds__(256) void rescale_combine_kernel(RescaleArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y;
  const PrimeConst pc = a.prime[i];
  const uint64_t* rs = a.tab + ((uint64_t)a.level * a.L + i) * 4;
  for (int comp = 0; comp < 2; ++comp) {
    const uint64_t cv = a.ct[blockIdx.z * a.ct_bstride + ((uint64_t)comp * (a.level + 1) + i) * a.n + c];
    const uint64_t wv = a.w[blockIdx.z * a.w_bstride + ((uint64_t)comp * a.level + i) * a.n + c];
    a.out[blockIdx.z * a.out_bstride + ((uint64_t)comp * a.level + i) * a.n + c] =
        sub_mod(reduce_2q(mul_shoup(cv, rs[0], rs[1], pc.q), pc.q), wv, pc.q);
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
  const uint64_t* y = a.b + blockIdx.z * a.in_bstride;
  uint64_t* d = a.out + blockIdx.z * a.out_bstride;
  const uint64_t a0 = x[off], a1 = x[lim + off], b0 = y[off], b1 = y[lim + off];
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
// blockIdx.y = limb i, blockIdx.z = o * n2 + g.
__global__ __launch_bounds__(256) void ptmac_kernel(PtMacArgs a) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y;
  const int o = blockIdx.z / a.n2, g = blockIdx.z % a.n2;
  const PrimeConst pc = a.prime[i];
  const uint64_t limbs = (uint64_t)(a.level + 1);
  const uint64_t off = (uint64_t)i * a.n + c;
  Acc3 s0 = {0, 0, 0}, s1 = {0, 0, 0};
  uint64_t r0 = 0, r1 = 0;
  int terms = 0;
  for (int ci = 0; ci < a.n_in; ++ci) {
    for (int b = 0; b < a.n1; ++b) {
      const uint64_t pt = a.diags[((((uint64_t)o * a.n_in + ci) * a.n2 + g) * a.n1 + b) * limbs * a.n + off];
      const uint64_t* ct = a.baby + ((uint64_t)b * a.n_in + ci) * 2 * limbs * a.n;
      const uint64_t c0 = ct[off], c1 = ct[limbs * a.n + off];
      const uint32_t pl = lo30(pt), ph = hi30(pt);
      acc3_mac(s0, pl, ph, lo30(c0), hi30(c0));
      acc3_mac(s1, pl, ph, lo30(c1), hi30(c1));
      if (++terms == 8) {  // fold every 8 terms
        r0 = add_mod(r0, acc3_reduce(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        r1 = add_mod(r1, acc3_reduce(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
        s0 = {0, 0, 0};
        s1 = {0, 0, 0};
        terms = 0;
      }
    }
  }
  r0 = add_mod(r0, acc3_reduce(s0, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
  r1 = add_mod(r1, acc3_reduce(s1, pc.q, pc.r64, pc.r64p, pc.inv1), pc.q);
  uint64_t* out = a.out + (uint64_t)blockIdx.z * 2 * limbs * a.n;
  out[off] = r0;
  out[limbs * a.n + off] = r1;
}

// out = x + y on [nl] limbs per item (limb i uses prime i).
__global__ void add_kernel(const uint64_t* x, const uint64_t* y, uint64_t* out, uint64_t bstride, int nl,
                           const PrimeConst* prime, int log_n) {
  const uint32_t c = blockIdx.x * blockDim.x + threadIdx.x;
  const int i = blockIdx.y % nl;
  const uint64_t off = blockIdx.z * bstride + ((uint64_t)blockIdx.y << log_n) + c;
  out[off] = add_mod(x[off], y[off], prime[i].q);
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
  hipLaunchKernelGGL(modup_kernel, dim3(c->N / 256, beta, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_inner_product(Ctx* c, hipStream_t s, IPArgs& a, int batch) {
  TraceScope ts(c, s, "inner_product", (double)batch * a.next * 2 * (a.beta + 1) * c->N);
  hipLaunchKernelGGL(inner_product_kernel, dim3(c->N / 256, a.next, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_moddown_conv(Ctx* c, hipStream_t s, ModDownArgs& a, int batch) {
  TraceScope ts(c, s, "moddown_conv", (double)batch * 2 * (a.K + (double)(a.level + 1) * (a.K + 1)) * c->N);
  hipLaunchKernelGGL(moddown_conv_kernel, dim3(c->N / 256, 2, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_combine(Ctx* c, hipStream_t s, CombineArgs& a, int batch) {
  TraceScope ts(c, s, "combine", (double)batch * 2 * (a.level + 1) * c->N);
  hipLaunchKernelGGL(combine_kernel, dim3(c->N / 256, a.level + 1, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_rescale_prep(Ctx* c, hipStream_t s, RescaleArgs& a, int batch) {
  TraceScope ts(c, s, "rescale", (double)batch * 2 * a.level * c->N);
  hipLaunchKernelGGL(rescale_prep_kernel, dim3(c->N / 256, 2, batch), dim3(256), 0, s, a);
  LAUNCH_CHECK();
  return CKKS_OK;
}

int launch_rescale_combine(Ctx* c, hipStream_t s, RescaleArgs& a, int batch) {
  TraceScope ts(c, s, "rescale", (double)batch * 2 * a.level * c->N);
  hipLaunchKernelGGL(rescale_combine_kernel, dim3(c->N / 256, a.level, batch), dim3(256), 0, s, a);
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
  hipLaunchKernelGGL(ptmac_kernel, dim3(c->N / 256, a.level + 1, n_out * a.n2), dim3(256), 0, s, a);
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

}  // namespace ckks
