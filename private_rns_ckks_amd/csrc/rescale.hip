// Rescale of a batch by its top limb q_l with the basis conversion fused
// into the forward NTT's column pass and the final combination into its row
// pass (the converted limbs make one round trip through memory instead of
// three).  Optionally a per-limb constant (a constant polynomial in NTT form)
// is added to component 0, and another ciphertext to the output, by the same
// final store.  Per item,
// component and limb i < l, with v = iNTT(c_l) canonical and vbar its centred
// lift:
//   w_i   = (vbar mod q_i) * [q_l^-1]_{q_i}
//   out_i = c_i * [q_l^-1]_{q_i} - NTT(w_i)          (mod q_i)
#include <string.h>

#include "kernels.h"
#include "ntt_core.h"

namespace ckks {

namespace {

using namespace nttc;

struct RescalePassArgs {
  const uint64_t* v;   // item b: v + b*v_bstride, [2][N] iNTT of limb l
  uint64_t* w;         // item b: w + b*w_bstride, [2][l][N]
  const uint64_t* ct;  // item b: ct + b*ct_bstride, [2][l+1][N]
  uint64_t* out;       // item b: out + b*out_bstride, [2][l][N]
  const uint64_t* acc; // optional, added to the output: item b at acc + b*acc_bstride, [2][l][N]
  uint64_t v_bstride, w_bstride, ct_bstride, out_bstride, acc_bstride;
  const uint64_t* tab;  // [L][L][4]: for level l, limb i: {q_l^-1, Shoup, q_l mod q_i, 0}
  const PrimeConst* prime;
  const uint64_t* tw;  // forward twiddles
  int log_n, level, L;
  int has_add;
  uint64_t add0[64];  // has_add: added to component 0 of limb i (a constant in NTT form)
};

// Column-pass input: w_i computed from v on load.
struct PrepIO {
  typedef NoOps Ops;
  const uint64_t* v;
  uint64_t* dst;
  uint64_t q, inv1, qinv, qinvp, qlmod, half;
  __device__ __forceinline__ uint64_t load(uint32_t j) const {
    const uint64_t x = v[j];
    uint64_t t = x >= q ? reduce64(x, q, inv1) : x;
    if (x > half) t = sub_mod(t, qlmod, q);
    return reduce_2q(mul_shoup(t, qinv, qinvp, q), q);
  }
  __device__ __forceinline__ void after_load(uint32_t, uint64_t) const {}
  __device__ __forceinline__ Ops fetch(uint32_t) const { return Ops(); }
  __device__ __forceinline__ void store(uint32_t j, uint64_t x, const Ops&) const { dst[j] = x; }
};

template <int RA, int RB, int LOGN>
__global__ __launch_bounds__(kThreads) void rescale_col_kernel(RescalePassArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<true, RB, ROWS>()];
  const int job = blockIdx.y, item = blockIdx.z;  // job = comp * l + i
  const int comp = job / a.level, i = job % a.level;
  const PrimeConst& pc = a.prime[i];
  const uint64_t* rs = a.tab + ((uint64_t)a.level * a.L + i) * 4;
  PrepIO io;
  io.v = a.v + item * a.v_bstride + ((uint64_t)comp << a.log_n);
  io.dst = a.w + item * a.w_bstride + ((uint64_t)job << a.log_n);
  io.q = pc.q;
  io.inv1 = pc.inv1;
  io.qinv = rs[0];
  io.qinvp = rs[1];
  io.qlmod = rs[2];
  io.half = (a.prime[a.level].q - 1) / 2;
  Finish fin{0, 0, 0, pc.inv1};
  run_pass<RA, RB, false, true, LOGN>(io, lds, blockIdx.x, a.log_n, a.tw + ((uint64_t)i << (a.log_n + 1)), pc.q,
                                      fin);
}

// Row-pass output: c_i * q_l^-1 - NTT(w_i) (+ constant) (+ acc).  With acc
// equal to out each word is read and written by the same thread.
struct CombOps {
  uint64_t c, a;
};
struct RescaleCombineIO {
  typedef CombOps Ops;
  const uint64_t* w;
  const uint64_t* ct;
  const uint64_t* acc;
  uint64_t* out;
  uint64_t q, qinv, qinvp, add;
  __device__ __forceinline__ uint64_t load(uint32_t j) const { return w[j]; }
  __device__ __forceinline__ void after_load(uint32_t, uint64_t) const {}
  __device__ __forceinline__ Ops fetch(uint32_t j) const { return Ops{ct[j], acc ? acc[j] : 0}; }
  __device__ __forceinline__ void store(uint32_t j, uint64_t x, const Ops& o) const {
    out[j] = add_mod(add_mod(sub_mod(reduce_2q(mul_shoup(o.c, qinv, qinvp, q), q), x, q), add, q), o.a, q);
  }
};

template <int RA, int RB, int LOGN>
__global__ __launch_bounds__(kThreads) void rescale_row_kernel(RescalePassArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<false, RB, ROWS>()];
  const GridPos gp = row_grid_pos();
  const int job = gp.job, item = gp.item;
  const int comp = job / a.level, i = job % a.level;
  const PrimeConst& pc = a.prime[i];
  const uint64_t* rs = a.tab + ((uint64_t)a.level * a.L + i) * 4;
  RescaleCombineIO io;
  io.w = a.w + item * a.w_bstride + ((uint64_t)job << a.log_n);
  io.ct = a.ct + item * a.ct_bstride + ((uint64_t)(comp * (a.level + 1) + i) << a.log_n);
  io.out = a.out + item * a.out_bstride + ((uint64_t)job << a.log_n);
  io.acc = a.acc ? a.acc + item * a.acc_bstride + ((uint64_t)job << a.log_n) : nullptr;
  io.q = pc.q;
  io.qinv = rs[0];
  io.qinvp = rs[1];
  io.add = (a.has_add && comp == 0) ? a.add0[i] : 0;
  Finish fin{1, 0, 0, pc.inv1};
  run_pass<RA, RB, false, false, LOGN>(io, lds, gp.tile, a.log_n, a.tw + ((uint64_t)i << (a.log_n + 1)), pc.q, fin);
}

}  // namespace

int rescale_fused(Ctx* c, hipStream_t s, const uint64_t* ct, uint64_t ct_bstride, const uint64_t* v, uint64_t v_bstride,
                  uint64_t* w, uint64_t w_bstride, uint64_t* out, uint64_t out_bstride, int batch, int level,
                  const uint64_t* add0, const uint64_t* acc, uint64_t acc_bstride) {
  const uint32_t N = c->N;
  const int log_n = (int)c->log_n;
  const int lr = logb_row(log_n), lc = logb_col(log_n);
  RescalePassArgs a;
  memset(&a, 0, sizeof(a));
  a.v = v;
  a.w = w;
  a.ct = ct;
  a.out = out;
  a.v_bstride = v_bstride;
  a.w_bstride = w_bstride;
  a.ct_bstride = ct_bstride;
  a.out_bstride = out_bstride;
  a.tab = c->d_rescale;
  a.prime = c->d_prime;
  a.tw = c->d_tw_fwd;
  a.log_n = log_n;
  a.level = level;
  a.L = (int)c->L;
  a.acc = acc;
  a.acc_bstride = acc_bstride;
  if (add0) {
    if (level > 64) return set_error(CKKS_EINTERNAL, "too many limbs for a fused constant");
    a.has_add = 1;
    for (int i = 0; i < level; ++i) a.add0[i] = add0[i];
  }
  auto fc = CKKS_PICK_PASS(rescale_col_kernel, log_n, lc);
  auto fr = CKKS_PICK_PASS(rescale_row_kernel, log_n, lr);
  if (!fc || !fr) return set_error(CKKS_EINTERNAL, "unsupported N");
  {
    TraceScope ts(c, s, "rescale", (double)batch * 2 * level * ((double)(N / 2) * lc + N));
    hipLaunchKernelGGL(fc, dim3(pass_tiles(N, lc), 2 * level, batch), dim3(kThreads), 0, s, a);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  {
    TraceScope ts(c, s, "rescale", (double)batch * 2 * level * ((double)(N / 2) * lr + N));
    hipLaunchKernelGGL(fr, dim3(pass_tiles(N, lr), 2 * level, batch), dim3(kThreads), 0, s, a);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  return CKKS_OK;
}

}  // namespace ckks
