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
  const uint64_t* scale_tab; // inverse final pass, scale_mode 2: {w, w'} pairs
  uint32_t log_n;
  uint32_t s0;               // first global stage handled by this pass
  uint32_t final_pass;       // reduce to [0,q) at the end
  uint32_t scale_mode;       // inverse final pass: 0 none, 1 times 1/N, 2 times scale_tab[scale_idx[job]]
  uint16_t src_limb[kMaxJobs];
  uint16_t dst_limb[kMaxJobs];
  uint16_t scale_idx[kMaxJobs];
  uint8_t prime_idx[kMaxJobs];
};

// global word index (within the limb) of tile element (row, col)
template <bool COLFAST>
__device__ __forceinline__ uint32_t tile_index(uint32_t tile, uint32_t row, uint32_t col, int logb, int log_n) {
  if (COLFAST) return tile * kCols + col + (row << (log_n - logb));
  return ((tile * kCols + col) << logb) + row;
}

// LDS position of tile element (row, col).  Column pass: row-major with 16
// padding words after every 2^RB rows; row pass: column-major with the low 4
// row bits XOR-ed with the next 4 and 16 padding words per column.  Both make
// the register rounds' 64-bit LDS accesses hit distinct bank pairs.
template <bool COLFAST, int RB, int ROWS>
__device__ __forceinline__ int lds_index(int row, int col) {
  if (COLFAST) return row * kCols + col + (row >> RB) * 16;
  return col * (ROWS + 16) + (row ^ ((row >> 4) & 15));
}
template <bool COLFAST, int RB, int ROWS>
constexpr int lds_words() {
  return COLFAST ? ROWS * kCols + (ROWS >> RB) * 16 : kCols * (ROWS + 16);
}

__device__ __forceinline__ void load_tw(const uint64_t* tw, uint32_t ti, uint64_t& w, uint64_t& wp) {
  const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(tw + 2 * ti);
  w = v.x;
  wp = v.y;
}

// Forward (Cooley-Tukey) butterfly.  Lazy form for q < 2^57: no correction,
// both outputs grow by at most 4q per stage, so 16 stages from [0, q) stay
// below 65q < 2^64.  Otherwise values are kept in [0, 8q).
template <bool LAZY>
__device__ __forceinline__ void ct_butterfly(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  const uint64_t four_q = 4 * q;
  uint64_t u = x;
  if (!LAZY) u = u >= four_q ? u - four_q : u;
  const uint64_t t = mul_shoup_lazy(y, w, wp, q);  // [0, 4q)
  x = u + t;
  y = u + four_q - t;
}

// Inverse (Gentleman-Sande) butterfly on values in [0, 4q).
__device__ __forceinline__ void gs_butterfly(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  const uint64_t four_q = 4 * q;
  const uint64_t s = x + y;
  const uint64_t d = x + four_q - y;
  x = s >= four_q ? s - four_q : s;
  y = mul_shoup_lazy(d, w, wp, q);
}

// R stages in registers on the 2^R words x[] of one thread; the words are
// rows base + (i << pos) of column col.  Global stage of sub-stage s is
// s0 + logb - pos - R + s.
template <int R, bool INV, bool LAZY, bool COLFAST>
__device__ __forceinline__ void round_regs(uint64_t (&x)[1 << R], int base, int pos, int col, int logb, uint32_t tile,
                                           uint32_t s0, int log_n, const uint64_t* tw, uint64_t q) {
  constexpr int E = 1 << R;
#pragma unroll
  for (int ss = 0; ss < R; ++ss) {
    const int s = INV ? (R - 1 - ss) : ss;
    const int half = E >> (s + 1);
    const int S = s0 + logb - pos - R + s;
#pragma unroll
    for (int g = 0; g < (1 << s); ++g) {
      const int i0 = g * 2 * half;
      const uint32_t j = tile_index<COLFAST>(tile, base + (i0 << pos), col, logb, log_n);
      uint64_t w, wp;
      load_tw(tw, (1u << S) + (j >> (log_n - S)), w, wp);
#pragma unroll
      for (int m = 0; m < half; ++m) {
        if (INV) gs_butterfly(x[i0 + m], x[i0 + m + half], w, wp, q);
        else ct_butterfly<LAZY>(x[i0 + m], x[i0 + m + half], w, wp, q);
      }
    }
  }
}

// Work item -> (column, base row) of a round covering row bits [pos, pos+R).
// Column pass: columns vary fastest across lanes (adjacent words in memory);
// row pass: the in-column index varies fastest.
template <bool COLFAST, int R, int LOGB>
__device__ __forceinline__ void item_coords(int item, int pos, int& col, int& base) {
  constexpr int nb = 1 << (LOGB - R);
  int b;
  if (COLFAST) {
    col = item % kCols;
    b = item / kCols;
  } else {
    b = item % nb;
    col = item / nb;
  }
  base = ((b >> pos) << (pos + R)) | (b & ((1 << pos) - 1));
}

template <int RA, int RB, bool INV, bool COLFAST, bool LAZY>
__device__ __forceinline__ void pass_body(const PassArgs& a, uint64_t* lds, const uint64_t* src, uint64_t* dst,
                                          const uint64_t* tw, uint64_t q, int job) {
  constexpr int LOGB = RA + RB;
  constexpr int ROWS = 1 << LOGB;
  constexpr int TILE = ROWS * kCols;
  const uint32_t tile = blockIdx.x;
  const int log_n = a.log_n;
  const uint32_t s0 = a.s0;
  const int tid = threadIdx.x;
  // first round: forward = high bits (pos RB, RA stages); inverse = low bits (pos 0, RB stages)
  constexpr int R1 = INV ? RB : RA;
  constexpr int R2 = INV ? RA : RB;
  const int pos1 = INV ? 0 : RB;
  const int pos2 = INV ? RB : 0;
  // row-pass inverse: the first round's words are strided in memory; stage through LDS
  constexpr bool stage_in = INV && !COLFAST;
  // row-pass forward: the last round's words are strided in memory; stage through LDS
  constexpr bool stage_out = !INV && !COLFAST;
  if (stage_in) {
    for (int e = tid; e < TILE; e += kThreads) {
      const int row = e % ROWS, col = e / ROWS;
      lds[lds_index<COLFAST, RB, ROWS>(row, col)] = src[tile_index<COLFAST>(tile, row, col, LOGB, log_n)];
    }
    __syncthreads();
  }
  if (tid < kCols * (ROWS >> R1)) {
    int col, base;
    item_coords<COLFAST, R1, LOGB>(tid, pos1, col, base);
    uint64_t x[1 << R1];
#pragma unroll
    for (int i = 0; i < (1 << R1); ++i) {
      const int row = base + (i << pos1);
      x[i] = stage_in ? lds[lds_index<COLFAST, RB, ROWS>(row, col)]
                      : src[tile_index<COLFAST>(tile, row, col, LOGB, log_n)];
    }
    round_regs<R1, INV, LAZY, COLFAST>(x, base, pos1, col, LOGB, tile, s0, log_n, tw, q);
    // each thread writes back exactly the words it read: no hazard with other threads
#pragma unroll
    for (int i = 0; i < (1 << R1); ++i) lds[lds_index<COLFAST, RB, ROWS>(base + (i << pos1), col)] = x[i];
  }
  __syncthreads();
  if (tid < kCols * (ROWS >> R2)) {
    int col, base;
    item_coords<COLFAST, R2, LOGB>(tid, pos2, col, base);
    uint64_t x[1 << R2];
#pragma unroll
    for (int i = 0; i < (1 << R2); ++i) x[i] = lds[lds_index<COLFAST, RB, ROWS>(base + (i << pos2), col)];
    round_regs<R2, INV, LAZY, COLFAST>(x, base, pos2, col, LOGB, tile, s0, log_n, tw, q);
    if (a.final_pass) {
      if (INV) {
        if (a.scale_mode) {
          uint64_t w, wp;
          if (a.scale_mode == 1) {
            const PrimeConst& pc = a.prime[a.prime_idx[job]];
            w = pc.ninv;
            wp = pc.ninvp;
          } else {
            w = a.scale_tab[2 * a.scale_idx[job]];
            wp = a.scale_tab[2 * a.scale_idx[job] + 1];
          }
#pragma unroll
          for (int i = 0; i < (1 << R2); ++i) x[i] = reduce_4q(mul_shoup_lazy(x[i], w, wp, q), q);
        } else {
#pragma unroll
          for (int i = 0; i < (1 << R2); ++i) x[i] = reduce_4q(x[i], q);
        }
      } else {
        const uint64_t inv1 = a.prime[a.prime_idx[job]].inv1;
#pragma unroll
        for (int i = 0; i < (1 << R2); ++i) x[i] = reduce64(x[i], q, inv1);
      }
    }
    if (stage_out) {
#pragma unroll
      for (int i = 0; i < (1 << R2); ++i) lds[lds_index<COLFAST, RB, ROWS>(base + (i << pos2), col)] = x[i];
    } else {
#pragma unroll
      for (int i = 0; i < (1 << R2); ++i) dst[tile_index<COLFAST>(tile, base + (i << pos2), col, LOGB, log_n)] = x[i];
    }
  }
  if (stage_out) {
    __syncthreads();
    for (int e = tid; e < TILE; e += kThreads) {
      const int row = e % ROWS, col = e / ROWS;
      dst[tile_index<COLFAST>(tile, row, col, LOGB, log_n)] = lds[lds_index<COLFAST, RB, ROWS>(row, col)];
    }
  }
}

template <int RA, int RB, bool INV, bool COLFAST>
__global__ __launch_bounds__(kThreads) void ntt_pass_kernel(PassArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<COLFAST, RB, ROWS>()];
  const int job = blockIdx.y;
  const int log_n = a.log_n;
  const uint64_t* src = a.src + blockIdx.z * a.src_bstride + (uint64_t)a.src_limb[job] * (1u << log_n);
  uint64_t* dst = a.dst + blockIdx.z * a.dst_bstride + (uint64_t)a.dst_limb[job] * (1u << log_n);
  const int p = a.prime_idx[job];
  const uint64_t q = a.prime[p].q;
  const uint64_t* tw = a.tw + ((uint64_t)p << (log_n + 1));
  if (!INV && q < (1ull << 57))
    pass_body<RA, RB, INV, COLFAST, true>(a, lds, src, dst, tw, q, job);
  else
    pass_body<RA, RB, INV, COLFAST, false>(a, lds, src, dst, tw, q, job);
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
  TraceScope ts(c, s, "ntt_pass", limbs * (c->N / 2) * logb + ((inv && a.final_pass && a.scale_mode) ? limbs * c->N : 0));
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
  a.scale_mode = scale ? 1u : 0u;
  a.scale_tab = nullptr;
  for (int i = 0; i < jobs.n; ++i) {
    a.src_limb[i] = jobs.src_limb[i];
    a.dst_limb[i] = jobs.dst_limb[i];
    a.prime_idx[i] = jobs.prime[i];
    a.scale_idx[i] = 0;
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
