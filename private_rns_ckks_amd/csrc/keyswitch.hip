// Hybrid key switching, with the automorphism fused into the first inverse
// NTT pass and the final combination fused into the last forward NTT pass.
//
// Per batch item, at level l (nq = l+1 ciphertext limbs, K special limbs,
// beta digits):
//   A  inverse row pass of the input polynomial; when rotating, the load
//      gathers tau_g(c1) (NTT form) and also writes it out for step E
//   B  inverse column pass; its final multiply uses [qhat_i^-1 N^-1]_{q_i},
//      so it produces the ModUp inputs y_i directly
//   C  ModUp conversion sum_i y_i [qhat_i]_{m_t} mod m_t to every target limb
//      t of every digit, then both forward NTT passes of those limbs
//   E  inner product with the key digits (digit limbs read the NTT-form input)
//   F  inverse NTT of the special limbs of both accumulators, final multiply
//      by [phat_k^-1 N^-1]_{p_k}: the ModDown inputs y_k
//   H  ModDown conversion sum_k y_k [1/p_k]_{q_i} - #{k: y_k > (p_k-1)/2}
//      (the centred lift, times P^-1), then the forward column pass
//   I  forward row pass whose store forms acc*P^-1 - NTT(w) (+ tau_g(c0))
//      (+ the input, when accumulating) straight into the output
#include <string.h>

#include "automorph.h"
#include "kernels.h"
#include "ntt_core.h"

namespace ckks {

namespace {

using namespace nttc;

// ---------------------------------------------------------------------------
// A: inverse row pass with optional automorphism gather and side output
struct GatherIO {
  typedef NoOps Ops;
  const uint64_t* src;
  uint64_t* side;
  uint64_t* dst;
  uint32_t g;
  int log_n;
  __device__ __forceinline__ uint64_t load(uint32_t j) const { return g ? src[automorph_src(j, g, log_n)] : src[j]; }
  __device__ __forceinline__ void after_load(uint32_t j, uint64_t v) const {
    if (side) side[j] = v;
  }
  __device__ __forceinline__ Ops fetch(uint32_t) const { return Ops(); }
  __device__ __forceinline__ void store(uint32_t j, uint64_t v, const Ops&) const { dst[j] = v; }
};

struct GatherArgs {
  const uint64_t* src;  // item b: src + b*src_bstride, limb i at + i*N
  uint64_t* side;       // gathered copy (NTT form) or NULL
  uint64_t* dst;
  uint64_t src_bstride, side_bstride, dst_bstride;
  const uint64_t* tw;
  const PrimeConst* prime;
  uint32_t g[kMaxChunk];
  int log_n;
};

template <int RA, int RB>
__global__ __launch_bounds__(kThreads) void intt_row_gather_kernel(GatherArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<false, RB, ROWS>()];
  const int limb = blockIdx.y, item = blockIdx.z;
  const uint64_t off = (uint64_t)limb << a.log_n;
  GatherIO io;
  io.src = a.src + item * a.src_bstride + off;
  io.side = a.side ? a.side + item * a.side_bstride + off : nullptr;
  io.dst = a.dst + item * a.dst_bstride + off;
  io.g = a.g[item];
  io.log_n = a.log_n;
  const PrimeConst& pc = a.prime[limb];
  Finish fin{0, 0, 0, pc.inv1};
  run_pass<RA, RB, true, false>(io, lds, blockIdx.x, a.log_n, (uint32_t)logb_col(a.log_n),
                                a.tw + ((uint64_t)limb << (a.log_n + 1)), pc.q, fin);
}

// ---------------------------------------------------------------------------
// I: forward row pass storing acc*P^-1 - v (+ gathered add) (+ accum)
struct CombineOps {
  uint64_t acc, add, accum;
};

struct CombineIO {
  typedef CombineOps Ops;
  const uint64_t* w;      // lazy column-pass output
  const uint64_t* acc;    // accumulator limb (NTT form)
  const uint64_t* add;    // or NULL
  const uint64_t* accum;  // or NULL
  uint64_t* out;
  uint64_t pinv, pinvp, q;
  uint32_t g;
  int log_n;
  __device__ __forceinline__ uint64_t load(uint32_t j) const { return w[j]; }
  __device__ __forceinline__ void after_load(uint32_t, uint64_t) const {}
  __device__ __forceinline__ Ops fetch(uint32_t j) const {
    Ops o;
    o.acc = acc[j];
    o.add = add ? add[g ? automorph_src(j, g, log_n) : j] : 0;
    o.accum = accum ? accum[j] : 0;
    return o;
  }
  __device__ __forceinline__ void store(uint32_t j, uint64_t v, const Ops& o) const {
    uint64_t r = sub_mod(reduce_4q(mul_shoup_lazy(o.acc, pinv, pinvp, q), q), v, q);
    r = add_mod(r, o.add, q);
    r = add_mod(r, o.accum, q);
    out[j] = r;
  }
};

struct CombinePassArgs {
  const uint64_t* w;    // item b: w + b*w_bstride, [2][nq][N]
  const uint64_t* acc;  // item b: acc + b*acc_bstride, [2][next][N]
  const uint64_t* add[2];
  const uint64_t* accum;
  uint64_t* out;
  uint64_t w_bstride, acc_bstride, add_bstride, accum_bstride, out_bstride;
  const uint64_t* pinv;  // [L][2]
  const uint64_t* tw;
  const PrimeConst* prime;
  uint32_t g[kMaxChunk];
  int log_n, nq, next, out_comp_limbs;
};

template <int RA, int RB>
__global__ __launch_bounds__(kThreads) void ntt_row_combine_kernel(CombinePassArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<false, RB, ROWS>()];
  const int job = blockIdx.y, item = blockIdx.z;  // job = comp * nq + i
  const int comp = job / a.nq, i = job % a.nq;
  const PrimeConst& pc = a.prime[i];
  CombineIO io;
  io.w = a.w + item * a.w_bstride + ((uint64_t)job << a.log_n);
  io.acc = a.acc + item * a.acc_bstride + ((uint64_t)(comp * a.next + i) << a.log_n);
  io.add = a.add[comp] ? a.add[comp] + item * a.add_bstride + ((uint64_t)i << a.log_n) : nullptr;
  io.accum = a.accum ? a.accum + item * a.accum_bstride + ((uint64_t)job << a.log_n) : nullptr;
  io.out = a.out + item * a.out_bstride + ((uint64_t)(comp * a.out_comp_limbs + i) << a.log_n);
  io.pinv = a.pinv[2 * i];
  io.pinvp = a.pinv[2 * i + 1];
  io.q = pc.q;
  io.g = a.g[item];
  io.log_n = a.log_n;
  Finish fin{1, 0, 0, pc.inv1};
  run_pass<RA, RB, false, false>(io, lds, blockIdx.x, a.log_n, (uint32_t)logb_col(a.log_n),
                                 a.tw + ((uint64_t)i << (a.log_n + 1)), pc.q, fin);
}

// ---------------------------------------------------------------------------
// launch helpers: kernel instance by pass size
#define PICK(kern, logb)                       \
  ((logb) == 5   ? kern<3, 2>                  \
   : (logb) == 6 ? kern<3, 3>                  \
   : (logb) == 7 ? kern<4, 3>                  \
   : (logb) == 8 ? kern<4, 4>                  \
                 : nullptr)

size_t ws_words(const Ctx* c, int level) {
  const size_t n = c->N, nq = level + 1, next = nq + c->K, beta = c->beta(level);
  return n * (nq /*T*/ + nq /*Y*/ + beta * next /*E*/ + 2 * next /*A*/ + 2 * nq /*W*/);
}

}  // namespace

size_t ks_ws_words(const Ctx* c, int level) { return ws_words(c, level); }

int ks_chunk(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, uint64_t d_stride,
             uint64_t add_stride, uint64_t accum_stride, uint64_t out_stride, int out_comp_limbs, uint64_t* ws) {
  const uint32_t N = c->N;
  const int log_n = (int)c->log_n;
  const int nq = level + 1, next = nq + (int)c->K, beta = c->beta(level);
  const uint64_t per = ws_words(c, level);
  uint64_t* T = ws;
  uint64_t* Y = T + (uint64_t)nq * N;
  uint64_t* E = Y + (uint64_t)nq * N;
  uint64_t* A = E + (uint64_t)beta * next * N;
  uint64_t* W = A + (uint64_t)2 * next * N;
  const int lr = logb_row(log_n), lc = logb_col(log_n);
  int rc;
  const bool rot = it[0].g != 0;

  // A: inverse row pass (gather tau_g(c1) when rotating)
  {
    GatherArgs ga;
    ga.src = it[0].d;
    ga.src_bstride = d_stride;
    ga.side = rot ? T : nullptr;
    ga.side_bstride = per;
    ga.dst = Y;
    ga.dst_bstride = per;
    ga.tw = c->d_tw_inv;
    ga.prime = c->d_prime;
    for (int i = 0; i < n_items; ++i) ga.g[i] = it[i].g;
    ga.log_n = log_n;
    auto fn = PICK(intt_row_gather_kernel, lr);
    if (!fn) return set_error(CKKS_EINTERNAL, "unsupported N");
    TraceScope ts(c, s, "ntt_pass", (double)n_items * nq * (N / 2) * lr);
    hipLaunchKernelGGL(fn, dim3(pass_tiles(N, lr), nq, n_items), dim3(kThreads), 0, s, ga);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  const uint64_t* Tsrc = rot ? T : it[0].d;
  const uint64_t T_stride = rot ? per : d_stride;
  // B: inverse column pass, times [qhat_i^-1 N^-1]: the ModUp inputs y_i
  {
    NttJobs jobs;
    uint32_t off[kMaxJobs];
    for (int j = 0; j < beta; ++j) {
      const ModUpEntry& en = c->modup[level][j];
      for (int i = en.lo; i < en.hi; ++i) {
        off[jobs.n] = (uint32_t)(en.offset + 2 * (i - en.lo));
        jobs.add(i, i, i);
      }
    }
    // the row pass above already ran: run only the column pass, in place on Y
    if ((rc = ntt_pass_only(c, s, Y, Y, per, per, n_items, jobs, true, false, 2, c->d_modup, off))) return rc;
  }
  // C: ModUp conversion, then both forward passes of the converted limbs
  {
    ModUpArgs mu;
    memset(&mu, 0, sizeof(mu));
    mu.x = Y;
    mu.out = E;
    mu.x_bstride = per;
    mu.out_bstride = per;
    mu.tables = c->d_modup;
    mu.prime = c->d_prime;
    mu.n = N;
    mu.level = level;
    mu.next = next;
    mu.L = (int)c->L;
    for (int j = 0; j < beta; ++j) {
      const ModUpEntry& en = c->modup[level][j];
      mu.lo[j] = en.lo;
      mu.hi[j] = en.hi;
      mu.offset[j] = en.offset;
    }
    if ((rc = launch_modup(c, s, mu, beta, n_items))) return rc;
    NttJobs jobs;
    for (int j = 0; j < beta; ++j)
      for (int t = 0; t < next; ++t) {
        if (t >= c->modup[level][j].lo && t < c->modup[level][j].hi) continue;
        jobs.add(j * next + t, j * next + t, c->ext_prime(level, t));
      }
    if ((rc = ntt_run(c, s, E, E, per, per, n_items, jobs, false, false))) return rc;
  }
  // E: inner product
  {
    IPArgs ip;
    memset(&ip, 0, sizeof(ip));
    ip.d = Tsrc;
    ip.ext = E;
    ip.acc = A;
    ip.d_bstride = T_stride;
    ip.ext_bstride = per;
    ip.acc_bstride = per;
    for (int i = 0; i < n_items; ++i) ip.evk[i] = it[i].evk;
    ip.prime = c->d_prime;
    ip.n = N;
    ip.level = level;
    ip.next = next;
    ip.beta = beta;
    ip.alpha = (int)c->alpha;
    ip.L = (int)c->L;
    ip.K = (int)c->K;
    if ((rc = launch_inner_product(c, s, ip, n_items))) return rc;
  }
  // F, G: inverse NTT of the special limbs, times [phat_k^-1 N^-1]: y_k
  {
    NttJobs jobs;
    uint32_t off[kMaxJobs];
    for (int comp = 0; comp < 2; ++comp)
      for (int k = 0; k < (int)c->K; ++k) {
        off[jobs.n] = (uint32_t)(c->md.phinv + 2 * k);
        jobs.add(comp * next + nq + k, comp * next + nq + k, (int)c->L + k);
      }
    if ((rc = ntt_run_scaled(c, s, A, A, per, per, n_items, jobs, true, 2, c->d_moddown, off))) return rc;
  }
  // H: ModDown conversion, then the forward column pass
  {
    ModDownArgs md;
    memset(&md, 0, sizeof(md));
    md.acc = A;
    md.w = W;
    md.acc_bstride = per;
    md.w_bstride = per;
    md.conv = c->d_moddown + c->md.conv;
    md.prime = c->d_prime;
    md.n = N;
    md.level = level;
    md.next = next;
    md.L = (int)c->L;
    md.K = (int)c->K;
    if ((rc = launch_moddown_conv(c, s, md, n_items))) return rc;
    NttJobs jobs;
    for (int comp = 0; comp < 2; ++comp)
      for (int i = 0; i < nq; ++i) jobs.add(comp * nq + i, comp * nq + i, i);
    if ((rc = ntt_pass_only(c, s, W, W, per, per, n_items, jobs, false, true, 0, nullptr, nullptr))) return rc;
  }
  // I: forward row pass with the final combination
  {
    CombinePassArgs ca;
    memset(&ca, 0, sizeof(ca));
    ca.w = W;
    ca.w_bstride = per;
    ca.acc = A;
    ca.acc_bstride = per;
    ca.add[0] = it[0].add[0];
    ca.add[1] = it[0].add[1];
    ca.add_bstride = add_stride;
    ca.accum = it[0].accum;
    ca.accum_bstride = accum_stride;
    ca.out = it[0].out;
    ca.out_bstride = out_stride;
    ca.pinv = c->d_moddown + c->md.pinv;
    ca.tw = c->d_tw_fwd;
    ca.prime = c->d_prime;
    for (int i = 0; i < n_items; ++i) ca.g[i] = it[i].add_g;
    ca.log_n = log_n;
    ca.nq = nq;
    ca.next = next;
    ca.out_comp_limbs = out_comp_limbs;
    auto fn = PICK(ntt_row_combine_kernel, lr);
    TraceScope ts(c, s, "ntt_pass", (double)n_items * 2 * nq * ((double)(N / 2) * lr + N));
    hipLaunchKernelGGL(fn, dim3(pass_tiles(N, lr), 2 * nq, n_items), dim3(kThreads), 0, s, ca);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  return CKKS_OK;
}

}  // namespace ckks
