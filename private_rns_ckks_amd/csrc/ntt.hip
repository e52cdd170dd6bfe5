// Batched negacyclic NTT / inverse NTT over a list of limb jobs (the
// transform itself is in ntt_core.h).
#include "ntt_core.h"
#include "rowpass.h"

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

// Inverse row pass (the transform's first pass) with the tile's inverse
// twiddles staged in LDS once per workgroup, over `items` batch items of one
// (tile, job).
template <int LOGB, int LOGN, int W>
__global__ __launch_bounds__((IPRounds<LOGB, W>::THREADS)) void ntt_row_inv_kernel(PassArgs a, int items,
                                                                                    int n_items) {
  typedef IPRounds<LOGB, W> G;
  __shared__ uint64_t lds[(1 << LOGB) * G::KC];
  __shared__ ulonglong2 twl[G::KC * ((1 << LOGB) - 1)];
  const GridPos g0 = row_grid_pos();
  const int job = g0.job;
  const int log_n = LOGN ? LOGN : (int)a.log_n;
  const int p = a.prime_idx[job];
  const PrimeConst& pc = a.prime[p];
  ip_stage_twiddles<LOGB, W>(twl, a.tw + ((uint64_t)p << (log_n + 1)), g0.tile, (uint32_t)logb_col(log_n));
  __syncthreads();  // every wave reads the twiddles every thread staged
  for (int k = 0; k < items; ++k) {
    const int item = g0.item * items + k;
    if (item >= n_items) break;
    const uint64_t* src = a.src + item * a.src_bstride + ((uint64_t)a.src_limb[job] << log_n);
    uint64_t* dst = a.dst + item * a.dst_bstride + ((uint64_t)a.dst_limb[job] << log_n);
    const int iar = inv_ar(pc.q);
    if (iar == AR_LAZY)
      ip_inv_row_pass<LOGB, AR_LAZY, W>(src, dst, lds, twl, g0.tile, pc.q, pc.inv1);
    else if (iar == AR_HARVEY)
      ip_inv_row_pass<LOGB, AR_HARVEY, W>(src, dst, lds, twl, g0.tile, pc.q, pc.inv1);
    else
      ip_inv_row_pass<LOGB, AR_STRICT, W>(src, dst, lds, twl, g0.tile, pc.q, pc.inv1);
  }
}

typedef void (*RowInvFn)(PassArgs, int, int);

// Words per thread of the inverse row pass (IPRounds).
constexpr int kRowInvW = 4;

RowInvFn pick_row_inv(int log_n, int logb) {
  if (log_n == 16 && logb == 8) return ntt_row_inv_kernel<8, 16, kRowInvW>;
  switch (logb) {
    case 5: return ntt_row_inv_kernel<5, 0, kRowInvW>;
    case 6: return ntt_row_inv_kernel<6, 0, kRowInvW>;
    case 7: return ntt_row_inv_kernel<7, 0, kRowInvW>;
    case 8: return ntt_row_inv_kernel<8, 0, kRowInvW>;
  }
  return nullptr;
}

// The inverse transform's row pass over `batch` items: up to 8 items per
// workgroup share the staged twiddles (C2's 16 polynomials per prime: 213.6
// against 236.6 us per inverse transform with the per-thread twiddle loads).
int launch_row_inv(Ctx* c, hipStream_t s, PassArgs& a, int batch, int njobs) {
  const int log_n = (int)c->log_n, logb = logb_row(log_n);
  RowInvFn fn = pick_row_inv(log_n, logb);
  if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
  const int items = std::max(1, std::min(8, batch / 2));
  const int logkc = ip_logkc(logb, kRowInvW);
  TraceScope ts(c, s, "ntt_pass", (double)njobs * batch * (c->N / 2) * logb);
  hipLaunchKernelGGL(fn, dim3(c->N >> (logkc + logb), njobs, (batch + items - 1) / items),
                     dim3((1u << (logkc + logb)) / kRowInvW), 0, s, a, items, batch);
  CKKS_HIP_CHECK(hipGetLastError());
  return CKKS_OK;
}

// Forward row pass (the transform's last pass, output in [0, q)) with the
// tile's twiddles staged in LDS once per workgroup, over `items` batch items
// of one (tile, job); 4 words per thread, so that four waves share a SIMD.
template <int LOGB, int LOGN>
__global__ __launch_bounds__((IPRounds<LOGB, 4>::THREADS)) void ntt_row_fwd_kernel(PassArgs a, int items,
                                                                                    int n_items) {
  typedef IPRounds<LOGB, 4> G;
  __shared__ uint64_t lds[(1 << LOGB) * G::KC];
  __shared__ ulonglong2 twl[G::KC * ((1 << LOGB) - 1)];
  const GridPos g0 = row_grid_pos();
  const int job = g0.job;
  const int log_n = LOGN ? LOGN : (int)a.log_n;
  const int p = a.prime_idx[job];
  const PrimeConst& pc = a.prime[p];
  const uint64_t q = pc.q;
  ip_stage_twiddles<LOGB, 4>(twl, a.tw + ((uint64_t)p << (log_n + 1)), g0.tile, (uint32_t)logb_col(log_n));
  __syncthreads();  // every wave reads the twiddles every thread staged
  int col, base;
  ip_item<G::RW, LOGB, 4>(0, 0, col, base);
  const uint32_t h0 = ip_word<LOGB, 4>(g0.tile, base, col) >> 1;
  const int far = fwd_ar(q);
  // lazy outputs lie below 70q < 2^63 for q < 2^57: one high-word quotient
  // leaves [0, 2q) when q is above 2^33 and below 2^56
  const bool hi_red = far == AR_LAZY && q > kReduceHiMin && q < (1ull << 56);
  for (int k = 0; k < items; ++k) {
    const int item = g0.item * items + k;
    if (item >= n_items) break;
    const uint64_t* src = a.src + item * a.src_bstride + ((uint64_t)a.src_limb[job] << log_n);
    ulonglong2* dst =
        reinterpret_cast<ulonglong2*>(a.dst + item * a.dst_bstride + ((uint64_t)a.dst_limb[job] << log_n));
    uint64_t x[4];
    if (far == AR_LAZY) {
      ip_row_pass_first<LOGB, AR_LAZY, 4>(src, lds, twl, g0.tile, log_n, q);
      ip_row_pass_rest<LOGB, AR_LAZY, 4>(x, lds, twl, g0.tile, log_n, q);
    } else if (far == AR_HARVEY) {
      ip_row_pass_first<LOGB, AR_HARVEY, 4>(src, lds, twl, g0.tile, log_n, q);
      ip_row_pass_rest<LOGB, AR_HARVEY, 4>(x, lds, twl, g0.tile, log_n, q);
    } else {
      ip_row_pass_first<LOGB, AR_STRICT, 4>(src, lds, twl, g0.tile, log_n, q);
      ip_row_pass_rest<LOGB, AR_STRICT, 4>(x, lds, twl, g0.tile, log_n, q);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = hi_red ? reduce_2q(reduce_hi(x[i], q, (uint32_t)pc.inv1), q) : reduce64(x[i], q, pc.inv1);
#pragma unroll
    for (int i = 0; i < 2; ++i) at_u32(dst, h0 + i) = make_ulonglong2(x[2 * i], x[2 * i + 1]);
  }
}

typedef void (*RowFwdFn)(PassArgs, int, int);

RowFwdFn pick_row_fwd(int log_n, int logb) {
  if (log_n == 16 && logb == 8) return ntt_row_fwd_kernel<8, 16>;
  switch (logb) {
    case 5: return ntt_row_fwd_kernel<5, 0>;
    case 6: return ntt_row_fwd_kernel<6, 0>;
    case 7: return ntt_row_fwd_kernel<7, 0>;
    case 8: return ntt_row_fwd_kernel<8, 0>;
  }
  return nullptr;
}

// The forward transform's row pass over `batch` items (final: output in [0, q)).
int launch_row_fwd(Ctx* c, hipStream_t s, PassArgs& a, int batch, int njobs) {
  const int log_n = (int)c->log_n, logb = logb_row(log_n);
  RowFwdFn fn = pick_row_fwd(log_n, logb);
  if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
  const int items = std::max(1, std::min(8, batch / 2));
  const int logkc = ip_logkc(logb, 4);
  TraceScope ts(c, s, "ntt_pass", (double)njobs * batch * (c->N / 2) * logb);
  hipLaunchKernelGGL(fn, dim3(c->N >> (logkc + logb), njobs, (batch + items - 1) / items),
                     dim3((1u << (logkc + logb)) / 4), 0, s, a, items, batch);
  CKKS_HIP_CHECK(hipGetLastError());
  return CKKS_OK;
}

typedef void (*PassFn)(PassArgs);

// Column pass (the forward transform's first pass, the inverse's last); the
// row passes run in ntt_row_fwd_kernel and ntt_row_inv_kernel.
int launch_col_pass(Ctx* c, hipStream_t s, PassArgs& a, int batch, int njobs, bool inv) {
  const int log_n = (int)c->log_n, logb = logb_col(log_n);
  PassFn fn = inv ? CKKS_PICK_PASS(ntt_pass_kernel, log_n, logb, true, true)
                  : CKKS_PICK_PASS(ntt_pass_kernel, log_n, logb, false, true);
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
    rc = launch_col_pass(c, s, a, batch, jobs.n, false);
  } else {
    rc = launch_row_inv(c, s, a, batch, jobs.n);
  }
  if (rc) return rc;
  a.src = dst;
  a.src_bstride = dst_bstride;
  for (int i = 0; i < jobs.n; ++i) a.src_limb[i] = jobs.dst_limb[i];
  a.final_pass = 1;
  if (!inverse) return launch_row_fwd(c, s, a, batch, jobs.n);
  return launch_col_pass(c, s, a, batch, jobs.n, true);
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
  // the column pass is the forward transform's first and the inverse's last
  if (inverse == first) return inverse ? launch_row_inv(c, s, a, batch, jobs.n) : launch_row_fwd(c, s, a, batch, jobs.n);
  return launch_col_pass(c, s, a, batch, jobs.n, inverse);
}

int ntt_run(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
            int batch, const NttJobs& jobs, bool inverse, bool scale) {
  return ntt_run_scaled(c, s, src, dst, src_bstride, dst_bstride, batch, jobs, inverse, scale ? 1 : 0, nullptr,
                        nullptr);
}

}  // namespace ckks
