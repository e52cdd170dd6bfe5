// Batched negacyclic NTT / inverse NTT over a list of limb jobs (the
// transform itself is in ntt_core.h).
#include "ntt_core.h"

namespace ckks {

namespace {

using namespace nttc;

struct PassArgs {
  const uint64_t* src;
  uint64_t* dst;
  uint64_t src_bstride, dst_bstride;
  const uint64_t* tw;        // [prime][N][2]
  const PrimeConst* prime;   // [L+K]
  const uint64_t* scale_tab; // scale_mode 2: {w, w'} at word offset scale_off[job]
  uint32_t log_n;
  uint32_t final_pass;       // reduce to [0,q) at the end
  uint32_t scale_mode;       // inverse final pass: 0 none, 1 times 1/N, 2 times the table entry
  uint16_t src_limb[kMaxJobs];
  uint16_t dst_limb[kMaxJobs];
  uint32_t scale_off[kMaxJobs];
  uint8_t prime_idx[kMaxJobs];
};

template <int RA, int RB, int LOGN, bool INV, bool COLFAST>
__global__ __launch_bounds__(kThreads) void ntt_pass_kernel(PassArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<COLFAST, RB, ROWS>()];
  GridPos gp;
  if (COLFAST) {  // column-pass twiddles are few and shared by every tile
    gp.tile = blockIdx.x;
    gp.job = blockIdx.y;
    gp.item = blockIdx.z;
  } else {
    gp = row_grid_pos();
  }
  const int job = gp.job;
  const int log_n = a.log_n;
  PlainIO io;
  io.src = a.src + gp.item * a.src_bstride + (uint64_t)a.src_limb[job] * (1u << log_n);
  io.dst = a.dst + gp.item * a.dst_bstride + (uint64_t)a.dst_limb[job] * (1u << log_n);
  const int p = a.prime_idx[job];
  const PrimeConst& pc = a.prime[p];
  const uint64_t* tw = a.tw + ((uint64_t)p << (log_n + 1));
  Finish fin;
  fin.mode = a.final_pass ? 1 : 0;
  fin.inv1 = pc.inv1;
  fin.w = fin.wp = 0;
  if (INV && a.final_pass && a.scale_mode) {
    fin.mode = 2;
    if (a.scale_mode == 1) {
      fin.w = pc.ninv;
      fin.wp = pc.ninvp;
    } else {
      fin.w = a.scale_tab[a.scale_off[job]];
      fin.wp = a.scale_tab[a.scale_off[job] + 1];
    }
  }
  run_pass<RA, RB, INV, COLFAST, LOGN>(io, lds, gp.tile, log_n, tw, pc.q, fin);
}

typedef void (*PassFn)(PassArgs);

int launch_pass(Ctx* c, hipStream_t s, PassArgs& a, int batch, int njobs, int logb, bool inv, bool colfast) {
  const int log_n = (int)c->log_n;
  PassFn fn = inv ? (colfast ? CKKS_PICK_PASS(ntt_pass_kernel, log_n, logb, true, true)
                             : CKKS_PICK_PASS(ntt_pass_kernel, log_n, logb, true, false))
                  : (colfast ? CKKS_PICK_PASS(ntt_pass_kernel, log_n, logb, false, true)
                             : CKKS_PICK_PASS(ntt_pass_kernel, log_n, logb, false, false));
  if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
  const double limbs = (double)njobs * batch;
  TraceScope ts(c, s, "ntt_pass", limbs * (c->N / 2) * logb + ((inv && a.final_pass && a.scale_mode) ? limbs * c->N : 0));
  hipLaunchKernelGGL(fn, dim3(pass_tiles(c->N, logb), njobs, batch), dim3(kThreads), 0, s, a);
  CKKS_HIP_CHECK(hipGetLastError());
  return CKKS_OK;
}

}  // namespace

int ntt_run_scaled(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
                   int batch, const NttJobs& jobs, bool inverse, int scale_mode, const uint64_t* scale_tab,
                   const uint32_t* scale_off) {
  if (jobs.n == 0 || batch == 0) return CKKS_OK;
  if (jobs.n > kMaxJobs) return set_error(CKKS_EINTERNAL, "too many NTT jobs");
  const int log_n = (int)c->log_n;
  PassArgs a;
  a.tw = inverse ? c->d_tw_inv : c->d_tw_fwd;
  a.prime = c->d_prime;
  a.log_n = (uint32_t)log_n;
  a.scale_mode = (uint32_t)scale_mode;
  a.scale_tab = scale_tab;
  for (int i = 0; i < jobs.n; ++i) {
    a.src_limb[i] = jobs.src_limb[i];
    a.dst_limb[i] = jobs.dst_limb[i];
    a.prime_idx[i] = jobs.prime[i];
    a.scale_off[i] = scale_off ? scale_off[i] : 0;
  }
  // first pass: src -> dst; second pass in place on dst (dst limbs)
  a.src = src;
  a.dst = dst;
  a.src_bstride = src_bstride;
  a.dst_bstride = dst_bstride;
  a.final_pass = 0;
  int rc;
  if (!inverse) {
    rc = launch_pass(c, s, a, batch, jobs.n, logb_col(log_n), false, true);
  } else {
    rc = launch_pass(c, s, a, batch, jobs.n, logb_row(log_n), true, false);
  }
  if (rc) return rc;
  a.src = dst;
  a.src_bstride = dst_bstride;
  for (int i = 0; i < jobs.n; ++i) a.src_limb[i] = jobs.dst_limb[i];
  a.final_pass = 1;
  if (!inverse) {
    return launch_pass(c, s, a, batch, jobs.n, logb_row(log_n), false, false);
  }
  return launch_pass(c, s, a, batch, jobs.n, logb_col(log_n), true, true);
}

int ntt_pass_only(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
                  int batch, const NttJobs& jobs, bool inverse, bool first, int scale_mode, const uint64_t* scale_tab,
                  const uint32_t* scale_off) {
  if (jobs.n == 0 || batch == 0) return CKKS_OK;
  if (jobs.n > kMaxJobs) return set_error(CKKS_EINTERNAL, "too many NTT jobs");
  const int log_n = (int)c->log_n;
  PassArgs a;
  a.tw = inverse ? c->d_tw_inv : c->d_tw_fwd;
  a.prime = c->d_prime;
  a.log_n = (uint32_t)log_n;
  a.scale_mode = (uint32_t)scale_mode;
  a.scale_tab = scale_tab;
  for (int i = 0; i < jobs.n; ++i) {
    a.src_limb[i] = jobs.src_limb[i];
    a.dst_limb[i] = jobs.dst_limb[i];
    a.prime_idx[i] = jobs.prime[i];
    a.scale_off[i] = scale_off ? scale_off[i] : 0;
  }
  a.src = src;
  a.dst = dst;
  a.src_bstride = src_bstride;
  a.dst_bstride = dst_bstride;
  a.final_pass = first ? 0 : 1;
  const bool colpass = (inverse != first);  // forward first / inverse second
  return launch_pass(c, s, a, batch, jobs.n, colpass ? logb_col(log_n) : logb_row(log_n), inverse, colpass);
}

int ntt_run(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
            int batch, const NttJobs& jobs, bool inverse, bool scale) {
  return ntt_run_scaled(c, s, src, dst, src_bstride, dst_bstride, batch, jobs, inverse, scale ? 1 : 0, nullptr,
                        nullptr);
}

}  // namespace ckks
