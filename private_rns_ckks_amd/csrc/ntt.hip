// Negacyclic NTT / inverse NTT on gfx950.
//
// Transform (the reading used throughout): word j of the forward output is the
// input polynomial evaluated at psi^(2*brv(j)+1).  The forward transform is a
// chain of log N radix-2 Cooley-Tukey stages with the powers of psi merged
// into the twiddles (stage S, butterfly block b uses psi^brv(2^S + b)); the
// inverse is the Gentleman-Sande chain with psi^-brv(.) and a final 1/N.
//
// Decomposition.  A 2^16-word limb (512 KiB) does not fit the 160 KiB LDS of
// a CU, so the log N stages are split into two passes over HBM:
//   column pass: the first LOGB1 stages only pair words whose index agrees
//                modulo N/2^LOGB1, so each column of 2^LOGB1 words (stride
//                N/2^LOGB1) is independent;
//   row pass:    the remaining LOGB2 stages act inside contiguous blocks of
//                2^LOGB2 words.
// (The inverse runs the row pass first.)  A workgroup loads a tile of 16
// columns (column pass: 16 adjacent words per row -> 128-byte segments) or 16
// contiguous blocks (row pass) into LDS, runs its stages in two register
// rounds of radix 2^RA and 2^RB (each thread holds 2^R words and applies R
// stages in registers; one LDS exchange between the rounds), and writes the
// tile back with coalesced stores.
//
// Arithmetic is Harvey's lazy butterfly with Shoup multiplication by the
// twiddle: forward values stay in [0, 4q), inverse values in [0, 2q); the last
// pass reduces to [0, q) (and applies 1/N for the inverse when asked).
#include "arith.h"
#include "internal.h"

namespace ckks {

namespace {

constexpr int kCols = 16;
constexpr int kThreads = 256;

struct PassArgs {
  const uint64_t* src;
  uint64_t* dst;
  uint64_t src_bstride, dst_bstride;
  const uint64_t* tw;        // [prime][N][2]
  const PrimeConst* prime;   // [L+K]
  uint32_t log_n;
  uint32_t s0;               // first global stage handled by this pass
  uint32_t final_pass;       // reduce to [0,q) at the end
  uint32_t scale;            // inverse: multiply by 1/N at the end
  uint16_t src_limb[kMaxJobs];
  uint16_t dst_limb[kMaxJobs];
  uint8_t prime_idx[kMaxJobs];
};

// global word index (within the limb) of tile element (row, col)
template <bool COLFAST>
__device__ __forceinline__ uint32_t tile_index(uint32_t tile, uint32_t row, uint32_t col, int logb, int log_n) {
  if (COLFAST) return tile * kCols + col + (row << (log_n - logb));
  return ((tile * kCols + col) << logb) + row;
}

__device__ __forceinline__ void ct_butterfly(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  const uint64_t two_q = 2 * q;
  uint64_t u = x >= two_q ? x - two_q : x;
  uint64_t t = mul_shoup(y, w, wp, q);  // [0, 2q)
  x = u + t;
  y = u - t + two_q;
}

__device__ __forceinline__ void gs_butterfly(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  const uint64_t two_q = 2 * q;
  uint64_t s = x + y;
  uint64_t d = x - y + two_q;
  x = s >= two_q ? s - two_q : s;
  y = mul_shoup(d, w, wp, q);
}

// One register round: R stages on 2^R words per thread.  The round covers row
// bits [pos, pos+R) of the tile; global stage of in-register sub-stage s is
// s0 + logb - pos - R + s.
template <int R, bool INV, bool COLFAST>
__device__ __forceinline__ void ntt_round(uint64_t* lds, int item, int pos, int logb, uint32_t tile,
                                          const PassArgs& a, const uint64_t* tw, uint64_t q, bool last) {
  constexpr int E = 1 << R;
  const int col = item % kCols;
  const int b = item / kCols;
  const int base = ((b >> pos) << (pos + R)) | (b & ((1 << pos) - 1));
  uint64_t x[E];
#pragma unroll
  for (int i = 0; i < E; ++i) x[i] = lds[(base + (i << pos)) * kCols + col];
  const int log_n = a.log_n;
#pragma unroll
  for (int ss = 0; ss < R; ++ss) {
    const int s = INV ? (R - 1 - ss) : ss;
    const int half = E >> (s + 1);
    const int S = a.s0 + logb - pos - R + s;
#pragma unroll
    for (int g = 0; g < (1 << s); ++g) {
      const int i0 = g * 2 * half;
      const uint32_t j = tile_index<COLFAST>(tile, base + (i0 << pos), col, logb, log_n);
      const uint32_t ti = (1u << S) + (j >> (log_n - S));
      const uint64_t w = tw[2 * ti], wp = tw[2 * ti + 1];
#pragma unroll
      for (int m = 0; m < half; ++m) {
        if (INV) gs_butterfly(x[i0 + m], x[i0 + m + half], w, wp, q);
        else ct_butterfly(x[i0 + m], x[i0 + m + half], w, wp, q);
      }
    }
  }
  if (last && a.final_pass) {
    if (INV) {
      if (a.scale) {
        const PrimeConst pc = a.prime[a.prime_idx[blockIdx.y]];
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] = reduce_2q(mul_shoup(x[i], pc.ninv, pc.ninvp, q), q);
      } else {
#pragma unroll
        for (int i = 0; i < E; ++i) x[i] = reduce_2q(x[i], q);
      }
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) {
        uint64_t v = x[i] >= 2 * q ? x[i] - 2 * q : x[i];
        x[i] = reduce_2q(v, q);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < E; ++i) lds[(base + (i << pos)) * kCols + col] = x[i];
}

template <int RA, int RB, bool INV, bool COLFAST>
__global__ __launch_bounds__(kThreads) void ntt_pass_kernel(PassArgs a) {
  constexpr int LOGB = RA + RB;
  constexpr int ROWS = 1 << LOGB;
  constexpr int TILE = ROWS * kCols;
  __shared__ uint64_t lds[TILE];
  const uint32_t tile = blockIdx.x;
  const int job = blockIdx.y;
  const int log_n = a.log_n;
  const uint64_t* src = a.src + blockIdx.z * a.src_bstride + (uint64_t)a.src_limb[job] * (1u << log_n);
  uint64_t* dst = a.dst + blockIdx.z * a.dst_bstride + (uint64_t)a.dst_limb[job] * (1u << log_n);
  const int p = a.prime_idx[job];
  const uint64_t q = a.prime[p].q;
  const uint64_t* tw = a.tw + ((uint64_t)p << (log_n + 1));

  // coalesced load: consecutive threads take consecutive addresses
  for (int e = threadIdx.x; e < TILE; e += kThreads) {
    int row, col;
    if (COLFAST) { col = e % kCols; row = e / kCols; }
    else { row = e % ROWS; col = e / ROWS; }
    lds[row * kCols + col] = src[tile_index<COLFAST>(tile, row, col, LOGB, log_n)];
  }
  __syncthreads();
  if (!INV) {
    // high row bits first
    if (threadIdx.x < kCols * (ROWS >> RA)) ntt_round<RA, INV, COLFAST>(lds, threadIdx.x, RB, LOGB, tile, a, tw, q, false);
    __syncthreads();
    if (threadIdx.x < kCols * (ROWS >> RB)) ntt_round<RB, INV, COLFAST>(lds, threadIdx.x, 0, LOGB, tile, a, tw, q, true);
  } else {
    // low row bits first
    if (threadIdx.x < kCols * (ROWS >> RB)) ntt_round<RB, INV, COLFAST>(lds, threadIdx.x, 0, LOGB, tile, a, tw, q, false);
    __syncthreads();
    if (threadIdx.x < kCols * (ROWS >> RA)) ntt_round<RA, INV, COLFAST>(lds, threadIdx.x, RB, LOGB, tile, a, tw, q, true);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TILE; e += kThreads) {
    int row, col;
    if (COLFAST) { col = e % kCols; row = e / kCols; }
    else { row = e % ROWS; col = e / ROWS; }
    dst[tile_index<COLFAST>(tile, row, col, LOGB, log_n)] = lds[row * kCols + col];
  }
}

typedef void (*PassFn)(PassArgs);

template <bool INV, bool COLFAST>
PassFn pick(int logb) {
  switch (logb) {
    case 5: return ntt_pass_kernel<3, 2, INV, COLFAST>;
    case 6: return ntt_pass_kernel<3, 3, INV, COLFAST>;
    case 7: return ntt_pass_kernel<4, 3, INV, COLFAST>;
    case 8: return ntt_pass_kernel<4, 4, INV, COLFAST>;
  }
  return nullptr;
}

int launch_pass(Ctx* c, hipStream_t s, PassArgs& a, int batch, int njobs, int logb, bool inv, bool colfast) {
  PassFn fn = inv ? (colfast ? pick<true, true>(logb) : pick<true, false>(logb))
                  : (colfast ? pick<false, true>(logb) : pick<false, false>(logb));
  if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
  const uint32_t tiles = c->N / ((1u << logb) * kCols);
  const double limbs = (double)njobs * batch;
  TraceScope ts(c, s, "ntt_pass", limbs * (c->N / 2) * logb + ((inv && a.final_pass && a.scale) ? limbs * c->N : 0));
  hipLaunchKernelGGL(fn, dim3(tiles, njobs, batch), dim3(kThreads), 0, s, a);
  CKKS_HIP_CHECK(hipGetLastError());
  return CKKS_OK;
}

}  // namespace

int ntt_run(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
            int batch, const NttJobs& jobs, bool inverse, bool scale) {
  if (jobs.n == 0 || batch == 0) return CKKS_OK;
  if (jobs.n > kMaxJobs) return set_error(CKKS_EINTERNAL, "too many NTT jobs");
  const int log_n = (int)c->log_n;
  const int logb_col = (log_n + 1) / 2;  // column pass: first stages of the forward transform
  const int logb_row = log_n - logb_col;
  PassArgs a;
  a.tw = inverse ? c->d_tw_inv : c->d_tw_fwd;
  a.prime = c->d_prime;
  a.log_n = (uint32_t)log_n;
  a.scale = scale ? 1u : 0u;
  for (int i = 0; i < jobs.n; ++i) {
    a.src_limb[i] = jobs.src_limb[i];
    a.dst_limb[i] = jobs.dst_limb[i];
    a.prime_idx[i] = jobs.prime[i];
  }
  // first pass: src -> dst; second pass in place on dst (dst limbs)
  a.src = src;
  a.dst = dst;
  a.src_bstride = src_bstride;
  a.dst_bstride = dst_bstride;
  a.final_pass = 0;
  if (!inverse) {
    a.s0 = 0;
    int rc = launch_pass(c, s, a, batch, jobs.n, logb_col, false, true);
    if (rc) return rc;
  } else {
    a.s0 = (uint32_t)logb_col;
    int rc = launch_pass(c, s, a, batch, jobs.n, logb_row, true, false);
    if (rc) return rc;
  }
  a.src = dst;
  a.src_bstride = dst_bstride;
  for (int i = 0; i < jobs.n; ++i) a.src_limb[i] = jobs.dst_limb[i];
  a.final_pass = 1;
  if (!inverse) {
    a.s0 = (uint32_t)logb_col;
    return launch_pass(c, s, a, batch, jobs.n, logb_row, false, false);
  }
  a.s0 = 0;
  return launch_pass(c, s, a, batch, jobs.n, logb_col, true, true);
}

}  // namespace ckks
