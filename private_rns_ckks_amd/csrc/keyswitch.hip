// Hybrid key switching, with the automorphism fused into the first inverse
// NTT pass and the final combination fused into the last forward NTT pass.
//
// Per batch item, at level l (nq = l+1 ciphertext limbs, K special limbs,
// beta digits):
//   A  inverse row pass of the input polynomial; when rotating, the load
//      gathers tau_g(c1) (NTT form)
//   B  inverse column pass; its final multiply uses [qhat_i^-1 N^-1]_{q_i},
//      so it produces the ModUp inputs y_i directly
//   C  ModUp conversion sum_i y_i [qhat_i]_{m_t} mod m_t to every target limb
//      t of every digit, then the forward column pass of those limbs
//   D  forward row pass of the converted limbs fused with the inner product
//      against the key digits (limbs inside their own digit read the
//      NTT-form input, through tau_g when rotating)
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
// A: inverse row pass with optional automorphism gather
struct GatherIO {
  typedef NoOps Ops;
  const uint64_t* src;
  uint64_t* dst;
  uint32_t g;
  int log_n;
  __device__ __forceinline__ uint64_t load(uint32_t j) const { return g ? src[automorph_src(j, g, log_n)] : src[j]; }
  __device__ __forceinline__ void after_load(uint32_t, uint64_t) const {}
  __device__ __forceinline__ Ops fetch(uint32_t) const { return Ops(); }
  __device__ __forceinline__ void store(uint32_t j, uint64_t v, const Ops&) const { dst[j] = v; }
};

struct GatherArgs {
  const uint64_t* src;  // item b: src + b*src_bstride, limb i at + i*N
  uint64_t* dst;
  uint64_t src_bstride, dst_bstride;
  const uint64_t* tw;
  const PrimeConst* prime;
  uint32_t g[kMaxChunk];
  int log_n;
};

template <int RA, int RB, int LOGN>
__global__ __launch_bounds__(kThreads) void intt_row_gather_kernel(GatherArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<false, RB, ROWS>()];
  const GridPos gp = row_grid_pos();
  const int limb = gp.job, item = gp.item;
  const uint64_t off = (uint64_t)limb << a.log_n;
  GatherIO io;
  io.src = a.src + item * a.src_bstride + off;
  io.dst = a.dst + item * a.dst_bstride + off;
  io.g = a.g[item];
  io.log_n = a.log_n;
  const PrimeConst& pc = a.prime[limb];
  Finish fin{0, 0, 0, pc.inv1};
  run_pass<RA, RB, true, false, LOGN>(io, lds, gp.tile, a.log_n, a.tw + ((uint64_t)limb << (a.log_n + 1)), pc.q,
                                      fin);
}

// ---------------------------------------------------------------------------
// D+E: forward row pass of the converted limbs fused with the inner product.
// A workgroup owns target limb t on one row-pass tile and loops over the
// digits: the digit's NTT (or, for t inside the digit, the NTT-form input)
// ends in LDS, and every thread multiply-accumulates its words against the
// key digit in a coalesced order (keys are read exactly once).  Products are
// Montgomery products (a*b*2^-64, lazy in [0, 2m)), so one 64-bit register
// per word and component carries the sum; the 2^-64 factor is removed at the
// end by a Shoup multiplication with 2^64 mod m.
struct RowIPArgs {
  const uint64_t* E;  // item b: E + b*E_bstride, [beta][next][N] column-pass output
  const uint64_t* T;  // item b: T + b*T_bstride, [nq][N] NTT-form input
  uint64_t* acc;      // item b: acc + b*acc_bstride, [2][next][N]
  uint64_t E_bstride, T_bstride, acc_bstride;
  const uint64_t* evk[kMaxChunk];
  const uint64_t* tw;  // forward twiddles
  const PrimeConst* prime;
  int log_n, level, next, beta, alpha, L, K;
  uint32_t g[kMaxChunk];  // item b's input limbs are read through tau_g (0: as they are)
  int shared_key;  // every item uses the same key: order the grid items first
  int items_per_wg, n_items;  // a workgroup runs items z*items_per_wg .. (twiddles staged once)
};

// A workgroup's tile is KC columns of 2^LOGB rows (8 columns from 2^7 rows
// on, so several workgroups share a CU).  The row pass's LOGB stages run as
// register rounds of at most 3 stages, the last of exactly 3, so every thread
// holds 8 words in every round and ends with 8 consecutive words of one
// column: the layout the multiply phase reads the key digits in.
__host__ __device__ constexpr int ip_logkc(int logb) { return logb >= 7 ? 3 : 4; }

template <int LOGB>
struct IPRounds {
  static constexpr int R3 = 3;
  static constexpr int R2 = LOGB >= 6 ? 3 : LOGB - 3;
  static constexpr int R1 = LOGB - R2 - R3;  // 0 when two rounds suffice
  static constexpr int LOGKC = ip_logkc(LOGB);
  static constexpr int KC = 1 << LOGKC;
  static constexpr int THREADS = KC << (LOGB - 3);
};

// global word index (within the limb) of tile element (row, col)
template <int LOGB>
__device__ __forceinline__ uint32_t ip_word(uint32_t tile, int row, int col) {
  return ((tile * IPRounds<LOGB>::KC + col) << LOGB) + row;
}

// LDS position of row-pass tile element (row, col): column-major, with row
// bits 0-4 XOR-ed by (row bits 5-7) and (row bits 6-7) << 3.  For the rounds
// of 2, 3, 3 stages at row bits 6, 3, 0 every 64-bit access of a wave then
// shares its bank pair with at most one other lane.
template <int LOGB>
__device__ __forceinline__ int ip_lds(int row, int col) {
  return col * (1 << LOGB) + (row ^ (((row >> 6) & 3) << 3) ^ ((row >> 5) & 7));
}

// The row pass's twiddles for one tile, staged in LDS once per workgroup and
// used by every digit: relative stage d (global stage s0 + d) of column col
// needs entries col * 2^d .. col * 2^d + 2^d - 1 of a run of KC * 2^d
// consecutive table entries, stored from LDS entry KC * (2^d - 1) on.
template <int LOGB>
__device__ __forceinline__ void ip_stage_twiddles(ulonglong2* twl, const uint64_t* tw, uint32_t tile, uint32_t s0) {
  typedef IPRounds<LOGB> G;
  constexpr int ENTRIES = G::KC * ((1 << LOGB) - 1);
  for (int e = threadIdx.x; e < ENTRIES; e += G::THREADS) {
    const int d = 31 - __clz((e >> G::LOGKC) + 1);
    const uint32_t g = (1u << (s0 + d)) + (tile << (G::LOGKC + d)) + (uint32_t)(e - G::KC * ((1 << d) - 1));
    twl[e] = *reinterpret_cast<const ulonglong2*>(tw + 2 * (uint64_t)g);
  }
}

// R forward stages on the 2^R words of one item (rows base + (i << pos) of
// column col), twiddles from the LDS copy.
template <int R, int LOGB, bool LAZY>
__device__ __forceinline__ void ip_butterflies(uint64_t (&x)[1 << R], int base, int pos, int col, const ulonglong2* twl,
                                               uint64_t q) {
  constexpr int E = 1 << R;
#pragma unroll
  for (int s = 0; s < R; ++s) {
    const int half = E >> (s + 1);
    const int d = LOGB - pos - R + s;
#pragma unroll
    for (int g = 0; g < (1 << s); ++g) {
      const int i0 = g * 2 * half;
      const int row = base + (i0 << pos);
      const ulonglong2 w = twl[IPRounds<LOGB>::KC * ((1 << d) - 1) + (col << d) + (row >> (LOGB - d))];
#pragma unroll
      for (int m = 0; m < half; ++m) ct_butterfly<LAZY>(x[i0 + m], x[i0 + m + half], w.x, w.y, q);
    }
  }
}

// One register round of R forward stages on row bits [POS, POS+R): item k of
// the thread (k < 8 >> R) is tid + k * THREADS; its words are rows
// base + (i << POS) of column col, read from global memory (src) or LDS and
// left in LDS or in x[].
template <int R, int POS, int LOGB, bool LAZY, bool FROM_GLOBAL, bool TO_LDS>
__device__ __forceinline__ void ip_round(uint64_t (&x)[8], const uint64_t* src, uint64_t* lds, const ulonglong2* twl,
                                         uint32_t tile, int log_n, uint64_t q) {
  constexpr int T = IPRounds<LOGB>::THREADS;
  constexpr int NI = 8 >> R;
  uint64_t y[NI][1 << R];
  int col[NI], base[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    item_coords<false, R, LOGB>(threadIdx.x + k * T, POS, col[k], base[k]);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      const int row = base[k] + (i << POS);
      y[k][i] = FROM_GLOBAL ? src[ip_word<LOGB>(tile, row, col[k])] : lds[ip_lds<LOGB>(row, col[k])];
    }
  }
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    ip_butterflies<R, LOGB, LAZY>(y[k], base[k], POS, col[k], twl, q);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      if (TO_LDS) lds[ip_lds<LOGB>(base[k] + (i << POS), col[k])] = y[k][i];
      else x[(k << R) + i] = y[k][i];
    }
  }
}

template <int LOGB, int LOGN, bool LAZY>
__device__ __forceinline__ void row_ip_body(const RowIPArgs& a, uint64_t* lds, ulonglong2* twl, const PrimeConst& pc,
                                            int keyl, const GridPos& gp, bool stage) {
  typedef IPRounds<LOGB> G;
  const int log_n = LOGN ? LOGN : a.log_n;
  const uint32_t s0 = (uint32_t)logb_col(log_n);
  const int t = gp.job, item = gp.item;
  const uint32_t tile = gp.tile;
  const uint64_t q = pc.q, mp = pc.mprime;
  const uint64_t* tw = a.tw + ((uint64_t)keyl << (log_n + 1));
  const uint64_t LKN = (uint64_t)(a.L + a.K) << log_n;
  // this thread's 8 output words: rows base..base+7 of column col
  int col, base;
  item_coords<false, 3, LOGB>(threadIdx.x, 0, col, base);
  const uint32_t w0 = ip_word<LOGB>(tile, base, col);
  const uint64_t* evk = a.evk[item] + ((uint64_t)keyl << log_n) + w0;
  if (stage) ip_stage_twiddles<LOGB>(twl, tw, tile, s0);  // read after the barrier that opens each digit's transform
  // Montgomery products are below 2m, so four of them sum below 8m < 2^63
  uint64_t accb[8], acca[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accb[i] = acca[i] = 0;
  for (int j = 0; j < a.beta; ++j) {
    const bool in_digit = t >= j * a.alpha && t < (j + 1) * a.alpha && t <= a.level;
    uint64_t x[8];
    if (in_digit) {  // NTT-form input limb, in [0, q); a rotation gathers tau_g of it here
      const uint64_t* limb = a.T + item * a.T_bstride + ((uint64_t)t << log_n);
      const uint32_t g = a.g[item];
      if (g) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = limb[automorph_src(w0 + i, g, log_n)];
      } else {
        const ulonglong2* src = reinterpret_cast<const ulonglong2*>(limb + w0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const ulonglong2 v = src[i];
          x[2 * i] = v.x;
          x[2 * i + 1] = v.y;
        }
      }
    } else {  // forward row pass of the converted limb; outputs stay lazy (< 65q, or < 8q)
      const uint64_t* src = a.E + item * a.E_bstride + ((uint64_t)(j * a.next + t) << log_n);
      __syncthreads();  // the previous digit's last round has read the tile
      if constexpr (G::R1 > 0) {
        ip_round<G::R1, LOGB - G::R1, LOGB, LAZY, true, true>(x, src, lds, twl, tile, log_n, q);
        __syncthreads();
        ip_round<G::R2, G::R3, LOGB, LAZY, false, true>(x, src, lds, twl, tile, log_n, q);
      } else {
        ip_round<G::R2, G::R3, LOGB, LAZY, true, true>(x, src, lds, twl, tile, log_n, q);
      }
      __syncthreads();
      ip_round<G::R3, 0, LOGB, LAZY, false, false>(x, src, lds, twl, tile, log_n, q);
    }
    const ulonglong2* kb = reinterpret_cast<const ulonglong2*>(evk + (uint64_t)(2 * j) * LKN);
    const ulonglong2* ka = reinterpret_cast<const ulonglong2*>(evk + (uint64_t)(2 * j + 1) * LKN);
    ulonglong2 vb[4], va[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      vb[i] = kb[i];
      va[i] = ka[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      accb[2 * i] += mont_mul_lazy(x[2 * i], vb[i].x, q, mp);
      accb[2 * i + 1] += mont_mul_lazy(x[2 * i + 1], vb[i].y, q, mp);
      acca[2 * i] += mont_mul_lazy(x[2 * i], va[i].x, q, mp);
      acca[2 * i + 1] += mont_mul_lazy(x[2 * i + 1], va[i].y, q, mp);
    }
    if ((j & 3) == 3) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        accb[i] = reduce64(accb[i], q, pc.inv1);
        acca[i] = reduce64(acca[i], q, pc.inv1);
      }
    }
  }
  // remove the 2^-64 of the Montgomery products: times 2^64 mod m
  ulonglong2* ob = reinterpret_cast<ulonglong2*>(a.acc + item * a.acc_bstride + ((uint64_t)t << log_n) + w0);
  ulonglong2* oa = reinterpret_cast<ulonglong2*>(a.acc + item * a.acc_bstride + ((uint64_t)(a.next + t) << log_n) + w0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ulonglong2 vb, va;
    vb.x = reduce_4q(mul_shoup_lazy(accb[2 * i], pc.r64, pc.r64p, q), q);
    vb.y = reduce_4q(mul_shoup_lazy(accb[2 * i + 1], pc.r64, pc.r64p, q), q);
    va.x = reduce_4q(mul_shoup_lazy(acca[2 * i], pc.r64, pc.r64p, q), q);
    va.y = reduce_4q(mul_shoup_lazy(acca[2 * i + 1], pc.r64, pc.r64p, q), q);
    ob[i] = vb;
    oa[i] = va;
  }
}

// at most 168 VGPRs: three waves per SIMD (three workgroups per CU at 2^8 rows)
template <int LOGB, int LOGN>
__global__ __launch_bounds__(IPRounds<LOGB>::THREADS) __attribute__((amdgpu_waves_per_eu(3))) void ntt_row_ip_kernel(
    RowIPArgs a) {
  __shared__ uint64_t lds[(1 << LOGB) * IPRounds<LOGB>::KC];
  __shared__ ulonglong2 twl[IPRounds<LOGB>::KC * ((1 << LOGB) - 1)];
  const GridPos g0 = a.shared_key ? row_grid_pos<true>() : row_grid_pos<false>();
  const int t = g0.job;
  const int keyl = t <= a.level ? t : a.L + (t - a.level - 1);
  const PrimeConst& pc = a.prime[keyl];
  for (int k = 0; k < a.items_per_wg; ++k) {
    GridPos gp = g0;
    gp.item = g0.item * a.items_per_wg + k;
    if (gp.item >= a.n_items) break;
    if (pc.q < (1ull << 57))
      row_ip_body<LOGB, LOGN, true>(a, lds, twl, pc, keyl, gp, k == 0);
    else
      row_ip_body<LOGB, LOGN, false>(a, lds, twl, pc, keyl, gp, k == 0);
  }
}

typedef void (*RowIPFn)(RowIPArgs);

RowIPFn pick_row_ip(int log_n, int logb) {
  if (log_n == 16 && logb == 8) return ntt_row_ip_kernel<8, 16>;
  switch (logb) {
    case 5: return ntt_row_ip_kernel<5, 0>;
    case 6: return ntt_row_ip_kernel<6, 0>;
    case 7: return ntt_row_ip_kernel<7, 0>;
    case 8: return ntt_row_ip_kernel<8, 0>;
  }
  return nullptr;
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

template <int RA, int RB, int LOGN>
__global__ __launch_bounds__(kThreads) void ntt_row_combine_kernel(CombinePassArgs a) {
  constexpr int ROWS = 1 << (RA + RB);
  __shared__ uint64_t lds[lds_words<false, RB, ROWS>()];
  const GridPos gp = row_grid_pos();
  const int job = gp.job, item = gp.item;  // job = comp * nq + i
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
  run_pass<RA, RB, false, false, LOGN>(io, lds, gp.tile, a.log_n, a.tw + ((uint64_t)i << (a.log_n + 1)), pc.q,
                                       fin);
}

// ---------------------------------------------------------------------------
// Hoisted rotations.  The digits of c1 are raised to the extended basis and
// transformed once per input (ks_decompose: [beta][next][N], NTT form,
// canonical); every rotation then gathers tau_g of those limbs straight into
// the inner product, with no transform of its own.
struct IPGatherArgs {
  const uint64_t* E;  // the chunk's input: [beta][next][N] raised digits
  const uint64_t* T;  // the chunk's input: c1, [nq][N] (limbs inside their own digit)
  uint64_t* acc;      // item b: acc + b*acc_bstride, [2][next][N]
  uint64_t acc_bstride;
  const uint64_t* evk[kMaxChunk];
  uint32_t g[kMaxChunk];
  const PrimeConst* prime;
  int log_n, level, next, beta, alpha, L, K;
};

constexpr int kGatherWords = 4;  // consecutive output words per thread

// acc_b[t][w] = sum_j D_j[t][pi_g(w)] * evk_j.b[t][w] (and acc_a), D_j the
// raised digit j (c1 itself for limbs inside digit j), pi_g the NTT-form
// automorphism.  Lazy Montgomery products as in ntt_row_ip_kernel.
__global__ __launch_bounds__(256) void ip_gather_kernel(IPGatherArgs a) {
  const int t = blockIdx.y, item = blockIdx.z;
  const int keyl = t <= a.level ? t : a.L + (t - a.level - 1);
  const PrimeConst& pc = a.prime[keyl];
  const uint64_t q = pc.q, mp = pc.mprime;
  const int log_n = a.log_n;
  const uint32_t w0 = (blockIdx.x * blockDim.x + threadIdx.x) * kGatherWords;
  const uint32_t g = __builtin_amdgcn_readfirstlane(a.g[item]);
  const uint64_t LKN = (uint64_t)(a.L + a.K) << log_n;
  const uint64_t* evk = a.evk[item] + ((uint64_t)keyl << log_n) + w0;
  uint32_t src[kGatherWords];
#pragma unroll
  for (int i = 0; i < kGatherWords; ++i) src[i] = automorph_src(w0 + i, g, log_n);
  uint64_t accb[kGatherWords], acca[kGatherWords];
#pragma unroll
  for (int i = 0; i < kGatherWords; ++i) accb[i] = acca[i] = 0;
  for (int j = 0; j < a.beta; ++j) {
    const bool in_digit = t >= j * a.alpha && t < (j + 1) * a.alpha && t <= a.level;
    const uint64_t* d = in_digit ? a.T + ((uint64_t)t << log_n) : a.E + ((uint64_t)(j * a.next + t) << log_n);
    const ulonglong2* kb = reinterpret_cast<const ulonglong2*>(evk + (uint64_t)(2 * j) * LKN);
    const ulonglong2* ka = reinterpret_cast<const ulonglong2*>(evk + (uint64_t)(2 * j + 1) * LKN);
    uint64_t x[kGatherWords];
    ulonglong2 vb[kGatherWords / 2], va[kGatherWords / 2];
#pragma unroll
    for (int i = 0; i < kGatherWords; ++i) x[i] = d[src[i]];
#pragma unroll
    for (int i = 0; i < kGatherWords / 2; ++i) {
      vb[i] = kb[i];
      va[i] = ka[i];
    }
#pragma unroll
    for (int i = 0; i < kGatherWords / 2; ++i) {
      accb[2 * i] += mont_mul_lazy(x[2 * i], vb[i].x, q, mp);
      accb[2 * i + 1] += mont_mul_lazy(x[2 * i + 1], vb[i].y, q, mp);
      acca[2 * i] += mont_mul_lazy(x[2 * i], va[i].x, q, mp);
      acca[2 * i + 1] += mont_mul_lazy(x[2 * i + 1], va[i].y, q, mp);
    }
    if ((j & 3) == 3) {  // sums of up to 4 products below 2m stay below 8m < 2^63
#pragma unroll
      for (int i = 0; i < kGatherWords; ++i) {
        accb[i] = reduce64(accb[i], q, pc.inv1);
        acca[i] = reduce64(acca[i], q, pc.inv1);
      }
    }
  }
  ulonglong2* ob = reinterpret_cast<ulonglong2*>(a.acc + item * a.acc_bstride + ((uint64_t)t << log_n) + w0);
  ulonglong2* oa = reinterpret_cast<ulonglong2*>(a.acc + item * a.acc_bstride + ((uint64_t)(a.next + t) << log_n) + w0);
#pragma unroll
  for (int i = 0; i < kGatherWords / 2; ++i) {
    ulonglong2 vb, va;
    vb.x = reduce_4q(mul_shoup_lazy(accb[2 * i], pc.r64, pc.r64p, q), q);
    vb.y = reduce_4q(mul_shoup_lazy(accb[2 * i + 1], pc.r64, pc.r64p, q), q);
    va.x = reduce_4q(mul_shoup_lazy(acca[2 * i], pc.r64, pc.r64p, q), q);
    va.y = reduce_4q(mul_shoup_lazy(acca[2 * i + 1], pc.r64, pc.r64p, q), q);
    ob[i] = vb;
    oa[i] = va;
  }
}

// ---------------------------------------------------------------------------
size_t ws_words(const Ctx* c, int level) {
  const size_t n = c->N, nq = level + 1, next = nq + c->K, beta = c->beta(level);
  return n * (nq /*Y*/ + beta * next /*E*/ + 2 * next /*A*/ + 2 * nq /*W*/);
}

// Steps F to I for n_items accumulators A (item i at A + i*per, [2][next][N]
// NTT form) with W as the ModDown scratch: out = ModDown(acc) (+ add, gathered
// through add_g) (+ accum).
int ks_back(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, uint64_t* A, uint64_t* W, uint64_t per,
            uint64_t add_stride, uint64_t accum_stride, uint64_t out_stride, int out_comp_limbs) {
  const uint32_t N = c->N;
  const int log_n = (int)c->log_n;
  const int nq = level + 1, next = nq + (int)c->K;
  const int lr = logb_row(log_n);
  int rc;
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
    auto fn = CKKS_PICK_PASS(ntt_row_combine_kernel, log_n, lr);
    TraceScope ts(c, s, "ntt_row_combine", (double)n_items * 2 * nq * ((double)(N / 2) * lr + N));
    hipLaunchKernelGGL(fn, dim3(pass_tiles(N, lr), 2 * nq, n_items), dim3(kThreads), 0, s, ca);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  return CKKS_OK;
}

}  // namespace

size_t ks_ws_words(const Ctx* c, int level) { return ws_words(c, level); }

size_t ks_dec_words(const Ctx* c, int level) {
  const size_t nq = level + 1, next = nq + c->K;
  return (size_t)c->N * (nq /*Y*/ + c->beta(level) * next /*E*/);
}

size_t ks_back_words(const Ctx* c, int level) {
  const size_t nq = level + 1, next = nq + c->K;
  return (size_t)c->N * (2 * next /*A*/ + 2 * nq /*W*/);
}

int ks_decompose(Ctx* c, hipStream_t s, int level, int n_in, const uint64_t* c1, uint64_t c1_stride, uint64_t* dec,
                 uint64_t dec_stride) {
  const uint32_t N = c->N;
  const int log_n = (int)c->log_n;
  const int nq = level + 1, next = nq + (int)c->K, beta = c->beta(level);
  uint64_t* Y = dec;
  uint64_t* E = dec + (uint64_t)nq * N;
  const int lr = logb_row(log_n);
  int rc;
  if (n_in > kMaxChunk) return set_error(CKKS_EINTERNAL, "too many inputs to decompose at once");
  // inverse row pass of c1
  {
    GatherArgs ga;
    memset(&ga, 0, sizeof(ga));
    ga.src = c1;
    ga.src_bstride = c1_stride;
    ga.dst = Y;
    ga.dst_bstride = dec_stride;
    ga.tw = c->d_tw_inv;
    ga.prime = c->d_prime;
    ga.log_n = log_n;
    auto fn = CKKS_PICK_PASS(intt_row_gather_kernel, log_n, lr);
    if (!fn) return set_error(CKKS_EINTERNAL, "unsupported N");
    TraceScope ts(c, s, "intt_row_gather", (double)n_in * nq * (N / 2) * lr);
    hipLaunchKernelGGL(fn, dim3(pass_tiles(N, lr), nq, n_in), dim3(kThreads), 0, s, ga);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  // inverse column pass, times [qhat_i^-1 N^-1]: the ModUp inputs y_i
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
    if ((rc = ntt_pass_only(c, s, Y, Y, dec_stride, dec_stride, n_in, jobs, true, false, 2, c->d_modup, off)))
      return rc;
  }
  // ModUp, then the whole forward transform of the converted limbs (canonical)
  {
    ModUpArgs mu;
    memset(&mu, 0, sizeof(mu));
    mu.x = Y;
    mu.out = E;
    mu.x_bstride = dec_stride;
    mu.out_bstride = dec_stride;
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
    if ((rc = launch_modup(c, s, mu, beta, n_in))) return rc;
    NttJobs jobs;
    for (int j = 0; j < beta; ++j)
      for (int t = 0; t < next; ++t) {
        if (t >= c->modup[level][j].lo && t < c->modup[level][j].hi) continue;
        jobs.add(j * next + t, j * next + t, c->ext_prime(level, t));
      }
    if ((rc = ntt_pass_only(c, s, E, E, dec_stride, dec_stride, n_in, jobs, false, true, 0, nullptr, nullptr)))
      return rc;
    if ((rc = ntt_pass_only(c, s, E, E, dec_stride, dec_stride, n_in, jobs, false, false, 0, nullptr, nullptr)))
      return rc;
  }
  return CKKS_OK;
}

int ks_hoisted_chunk(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, const uint64_t* dec,
                     const uint64_t* c1, uint64_t out_stride, uint64_t* ws) {
  const uint32_t N = c->N;
  const int nq = level + 1, next = nq + (int)c->K, beta = c->beta(level);
  const uint64_t per = ks_back_words(c, level);
  uint64_t* A = ws;
  uint64_t* W = ws + (uint64_t)2 * next * N;
  {
    IPGatherArgs ip;
    memset(&ip, 0, sizeof(ip));
    ip.E = dec + (uint64_t)nq * N;
    ip.T = c1;
    ip.acc = A;
    ip.acc_bstride = per;
    for (int i = 0; i < n_items; ++i) {
      ip.evk[i] = it[i].evk;
      ip.g[i] = it[i].g;
    }
    ip.prime = c->d_prime;
    ip.log_n = (int)c->log_n;
    ip.level = level;
    ip.next = next;
    ip.beta = beta;
    ip.alpha = (int)c->alpha;
    ip.L = (int)c->L;
    ip.K = (int)c->K;
    TraceScope ts(c, s, "ip_gather", (double)n_items * next * N * (2.0 * beta + 2));
    hipLaunchKernelGGL(ip_gather_kernel, dim3(N / (256 * kGatherWords), next, n_items), dim3(256), 0, s, ip);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  return ks_back(c, s, level, n_items, it, A, W, per, 0, 0, out_stride, nq);
}

int ks_chunk(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, uint64_t d_stride,
             uint64_t add_stride, uint64_t accum_stride, uint64_t out_stride, int out_comp_limbs, uint64_t* ws) {
  const uint32_t N = c->N;
  const int log_n = (int)c->log_n;
  const int nq = level + 1, next = nq + (int)c->K, beta = c->beta(level);
  const uint64_t per = ws_words(c, level);
  uint64_t* Y = ws;
  uint64_t* E = Y + (uint64_t)nq * N;
  uint64_t* A = E + (uint64_t)beta * next * N;
  uint64_t* W = A + (uint64_t)2 * next * N;
  const int lr = logb_row(log_n), lc = logb_col(log_n);
  int rc;

  // A: inverse row pass (gather tau_g(c1) when rotating)
  {
    GatherArgs ga;
    ga.src = it[0].d;
    ga.src_bstride = d_stride;
    ga.dst = Y;
    ga.dst_bstride = per;
    ga.tw = c->d_tw_inv;
    ga.prime = c->d_prime;
    for (int i = 0; i < n_items; ++i) ga.g[i] = it[i].g;
    ga.log_n = log_n;
    auto fn = CKKS_PICK_PASS(intt_row_gather_kernel, log_n, lr);
    if (!fn) return set_error(CKKS_EINTERNAL, "unsupported N");
    TraceScope ts(c, s, "intt_row_gather", (double)n_items * nq * (N / 2) * lr);
    hipLaunchKernelGGL(fn, dim3(pass_tiles(N, lr), nq, n_items), dim3(kThreads), 0, s, ga);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  const uint64_t* Tsrc = it[0].d;
  const uint64_t T_stride = d_stride;
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
    if ((rc = ntt_pass_only(c, s, E, E, per, per, n_items, jobs, false, true, 0, nullptr, nullptr))) return rc;
  }
  // D+E: forward row pass fused with the inner product
  {
    RowIPArgs ip;
    memset(&ip, 0, sizeof(ip));
    ip.E = E;
    ip.E_bstride = per;
    ip.T = Tsrc;
    ip.T_bstride = T_stride;
    for (int i = 0; i < n_items; ++i) ip.g[i] = it[i].g;
    ip.acc = A;
    ip.acc_bstride = per;
    ip.shared_key = 1;
    for (int i = 0; i < n_items; ++i) {
      ip.evk[i] = it[i].evk;
      if (it[i].evk != it[0].evk) ip.shared_key = 0;
    }
    ip.tw = c->d_tw_fwd;
    ip.prime = c->d_prime;
    ip.log_n = log_n;
    ip.level = level;
    ip.next = next;
    ip.beta = beta;
    ip.alpha = (int)c->alpha;
    ip.L = (int)c->L;
    ip.K = (int)c->K;
    RowIPFn fn = pick_row_ip(log_n, lr);
    if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
    double units = 0;
    for (int j = 0; j < beta; ++j) {
      const int na = c->modup[level][j].hi - c->modup[level][j].lo;
      units += (double)(next - na) * (N / 2) * lr;  // butterflies
    }
    units += (double)next * N * (2.0 * beta + 2);  // products and final reductions
    TraceScope ts(c, s, "ntt_row_ip", units * n_items);
    const int logkc = ip_logkc(lr);
    // two items per workgroup: the tile's twiddles are staged once for both
    // (half the twiddle traffic); more items leave too few workgroups
    const int ipw = 2;
    ip.items_per_wg = ipw;
    ip.n_items = n_items;
    hipLaunchKernelGGL(fn, dim3(N >> (lr + logkc), next, (n_items + ipw - 1) / ipw), dim3(1u << (lr - 3 + logkc)), 0,
                       s, ip);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  return ks_back(c, s, level, n_items, it, A, W, per, add_stride, accum_stride, out_stride, out_comp_limbs);
}

}  // namespace ckks
