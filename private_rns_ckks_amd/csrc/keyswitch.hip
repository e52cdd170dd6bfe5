// Hybrid key switching.
//
// Per batch item, at level l (nq = l+1 ciphertext limbs, K special limbs,
// beta digits of alpha limbs), ks_chunk runs:
//   A  inverse row pass of the input polynomial; when rotating, the load
//      gathers tau_g(c1) (NTT form)
//   B  inverse column pass times [qhat_i^-1 N^-1]_{q_i}: the ModUp inputs y_i
//   C  ModUp conversion sum_i y_i [qhat_i]_{m_t} mod m_t to every target limb
//      t of every digit, then the forward column pass of those limbs
//   D  special limbs: forward row pass of the converted limbs fused with the
//      inner product against the key digits, then the inverse row pass of
//      both accumulator components on the same tile
//   G  inverse column pass of the special accumulators times
//      [phat_k^-1 N^-1]_{p_k}: the ModDown inputs y_k
//   H  ModDown conversion sum_k y_k [1/p_k]_{q_i} - #{k: y_k > (p_k-1)/2}
//      (the centred lift, times P^-1), then the forward column pass
//   I  ciphertext limbs: forward row pass of the converted limbs fused with
//      the inner product (limbs inside their own digit read the NTT-form
//      input, through tau_g when rotating), then the forward row pass of the
//      ModDown output on the same tile, storing acc*P^-1 - NTT(w)
//      (+ tau_g(c0)) (+ the input, when accumulating) straight into the
//      output: the ciphertext-limb accumulators never go to memory.
// Hoisted rotations run A-C and the forward row pass once per input
// (ks_decompose); per rotation, a gathered inner product over every limb
// (ip_gather_kernel) and ks_back: the inverse NTT of the special limbs, H,
// and a combining forward row pass.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <string>
#include <vector>

#include "automorph.h"
#include "kernels.h"
#include "ntt_core.h"
#include "rowpass.h"

namespace ckks {

namespace {

using namespace nttc;

// ---------------------------------------------------------------------------
// A: inverse row pass with optional automorphism gather
struct GatherArgs {
  const uint64_t* src;  // item b: src + b*src_bstride, limb i at + i*N
  uint64_t* dst;
  uint64_t src_bstride, dst_bstride;
  const uint64_t* tw;
  const PrimeConst* prime;
  uint32_t g[kMaxChunk];
  int log_n;
};

// A: the first pass (the row pass) of the inverse NTT of c1's limbs, read
// through tau_g, for up to 8 batch items per workgroup that share the tile's
// inverse twiddles staged in LDS (as the batched inverse NTT); the output
// (below 4q) goes to the scaled inverse column pass.
template <int LOGB, int LOGN, int W>
__global__ __launch_bounds__((IPRounds<LOGB, W>::THREADS)) void intt_row_gather_kernel(GatherArgs a, int items,
                                                                                      int n_items) {
  typedef IPRounds<LOGB, W> G;
  __shared__ uint64_t lds[(1 << LOGB) * G::KC];
  __shared__ ulonglong2 twl[G::KC * ((1 << LOGB) - 1)];
  const GridPos g0 = row_grid_pos();
  const int limb = g0.job;
  const int log_n = LOGN ? LOGN : a.log_n;
  const PrimeConst& pc = a.prime[limb];
  ip_stage_twiddles<LOGB, W>(twl, a.tw + ((uint64_t)limb << (log_n + 1)), g0.tile, (uint32_t)logb_col(log_n));
  __syncthreads();  // every wave reads the twiddles every thread staged
  const int iar = inv_ar(pc.q);
  const uint64_t off = (uint64_t)limb << log_n;
  for (int k = 0; k < items; ++k) {
    const int item = g0.item * items + k;
    if (item >= n_items) break;
    const uint64_t* src = a.src + item * a.src_bstride + off;
    uint64_t* dst = a.dst + item * a.dst_bstride + off;
    const uint32_t g = a.g[item];
    if (iar == AR_LAZY)
      ip_inv_row_pass<LOGB, AR_LAZY, W>(src, dst, lds, twl, g0.tile, pc.q, pc.inv1, g, log_n);
    else if (iar == AR_HARVEY)
      ip_inv_row_pass<LOGB, AR_HARVEY, W>(src, dst, lds, twl, g0.tile, pc.q, pc.inv1, g, log_n);
    else
      ip_inv_row_pass<LOGB, AR_STRICT, W>(src, dst, lds, twl, g0.tile, pc.q, pc.inv1, g, log_n);
  }
}

typedef void (*GatherFn)(GatherArgs, int, int);

// Words per thread of step A (IPRounds).
constexpr int kGatherW = 4;

// Step A over n_items items of nq limbs.
int launch_gather(Ctx* c, hipStream_t s, const GatherArgs& ga, int nq, int n_items) {
  const int log_n = (int)c->log_n, logb = logb_row(log_n);
  GatherFn fn = nullptr;
  if (log_n == 16 && logb == 8) fn = intt_row_gather_kernel<8, 16, kGatherW>;
  else if (logb == 5) fn = intt_row_gather_kernel<5, 0, kGatherW>;
  else if (logb == 6) fn = intt_row_gather_kernel<6, 0, kGatherW>;
  else if (logb == 7) fn = intt_row_gather_kernel<7, 0, kGatherW>;
  else if (logb == 8) fn = intt_row_gather_kernel<8, 0, kGatherW>;
  if (!fn) return set_error(CKKS_EINTERNAL, "unsupported N");
  const int items = std::max(1, std::min(8, n_items / 2));
  const int logkc = ip_logkc(logb, kGatherW);
  TraceScope ts(c, s, "intt_row_gather", (double)n_items * nq * (c->N / 2) * logb);
  hipLaunchKernelGGL(fn, dim3(c->N >> (logkc + logb), nq, (n_items + items - 1) / items),
                     dim3((1u << (logkc + logb)) / kGatherW), 0, s, ga, items, n_items);
  CKKS_HIP_CHECK(hipGetLastError());
  return CKKS_OK;
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
  int t0;          // target limb of grid job 0 (job j handles limb t0 + j)
};

// Multiply-accumulate of target limb t (tile gp.tile, item gp.item) over the
// digits: accb[i] / acca[i] receive sum_j x_j * evk_j.{b,a} for the thread's
// W words (rows base..base+W-1 of column col), x_j the forward row pass of the
// converted limb E[j][t] or, for t inside digit j, the NTT-form input limb
// (through tau_g when rotating).  Sums of Montgomery products, reduced every
// mont_fold(m) digits (below 9m); the factor 2^-64 is left in them.
template <int LOGB, int LOGN, int AR, int W = 8>
__device__ __forceinline__ void ip_accumulate(const RowIPArgs& a, uint64_t* lds, const ulonglong2* twl,
                                              const PrimeConst& pc, int keyl, const GridPos& gp, uint64_t (&accb)[W],
                                              uint64_t (&acca)[W]) {
  constexpr int H = W / 2;  // 16-byte words per thread
  const int log_n = LOGN ? LOGN : a.log_n;
  const int t = gp.job + a.t0, item = gp.item;
  const uint32_t tile = gp.tile;
  const uint64_t q = pc.q, mp = pc.mprime;
  const uint64_t LKN = (uint64_t)(a.L + a.K) << log_n;
  int col, base;
  ip_item<IPRounds<LOGB, W>::RW, LOGB, W>(0, 0, col, base);
  const uint32_t w0 = ip_word<LOGB, W>(tile, base, col), h0 = w0 >> 1;
  const uint64_t* evk = a.evk[item] + ((uint64_t)keyl << log_n);
#pragma unroll
  for (int i = 0; i < W; ++i) accb[i] = acca[i] = 0;
  const int fold = mont_fold(q);
  int since = 0;
  for (int j = 0; j < a.beta; ++j) {
    const bool in_digit = t >= j * a.alpha && t < (j + 1) * a.alpha && t <= a.level;
    uint64_t x[W];
    if (in_digit) {  // NTT-form input limb, in [0, q); a rotation gathers tau_g of it here
      const uint64_t* limb = a.T + item * a.T_bstride + ((uint64_t)t << log_n);
      const uint32_t g = a.g[item];
      if (g) {
#pragma unroll
        for (int i = 0; i < W; ++i) x[i] = at_u32(limb, automorph_src(w0 + i, g, log_n));
      } else {
        const ulonglong2* src = reinterpret_cast<const ulonglong2*>(limb);
#pragma unroll
        for (int i = 0; i < H; ++i) {
          const ulonglong2 v = at_u32(src, h0 + i);
          x[2 * i] = v.x;
          x[2 * i + 1] = v.y;
        }
      }
    }
    // one key component at a time: 16 registers of key words live, not 32;
    // the first component's words load during the row pass's later rounds
    const ulonglong2* kb = reinterpret_cast<const ulonglong2*>(evk + (uint64_t)(2 * j) * LKN);
    const ulonglong2* ka = reinterpret_cast<const ulonglong2*>(evk + (uint64_t)(2 * j + 1) * LKN);
    ulonglong2 vb[H];
    if (!in_digit) {  // forward row pass of the converted limb; outputs stay lazy (< 70q, or < 8q)
      const uint64_t* src = a.E + item * a.E_bstride + ((uint64_t)(j * a.next + t) << log_n);
      ip_row_pass_first<LOGB, AR, W>(src, lds, twl, tile, log_n, q);
#pragma unroll
      for (int i = 0; i < H; ++i) vb[i] = at_u32(kb, h0 + i);
      ip_row_pass_rest<LOGB, AR, W>(x, lds, twl, tile, log_n, q);
    } else {
#pragma unroll
      for (int i = 0; i < H; ++i) vb[i] = at_u32(kb, h0 + i);
    }
    {
#pragma unroll
      for (int i = 0; i < H; ++i) {
        accb[2 * i] += mont_mul_lazy(x[2 * i], vb[i].x, q, mp);
        accb[2 * i + 1] += mont_mul_lazy(x[2 * i + 1], vb[i].y, q, mp);
      }
    }
    {
      ulonglong2 v[H];
#pragma unroll
      for (int i = 0; i < H; ++i) v[i] = at_u32(ka, h0 + i);
#pragma unroll
      for (int i = 0; i < H; ++i) {
        acca[2 * i] += mont_mul_lazy(x[2 * i], v[i].x, q, mp);
        acca[2 * i + 1] += mont_mul_lazy(x[2 * i + 1], v[i].y, q, mp);
      }
    }
    if (++since == fold) {
      since = 0;
#pragma unroll
      for (int i = 0; i < W; ++i) {
        accb[i] = reduce64(accb[i], q, pc.inv1);
        acca[i] = reduce64(acca[i], q, pc.inv1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Inner product of the special limbs only (targets t = l+1 .. l+K), followed
// on the same tile by the first pass of their inverse NTT (the row pass); the
// inverse column pass (scaled for ModDown) completes it.
//
// The inverse row pass of one component: the thread's W words (rows
// base..base+W-1 of its column, below 4q, below 2q for AR_STRICT) go through
// the Gentleman-Sande stages of the low row bits in registers, then of the
// higher row bits in rounds through the LDS tile (the rounds of the forward
// pass in reverse order), and are stored below 4q for the column pass
// (inv_row_out).  Twiddles come from the inverse table in global memory.
template <int LOGB, int AR, int W, int POS>
__device__ __forceinline__ void ip_inv_rounds_up(uint64_t* lds, uint32_t tile, int log_n, uint32_t s0,
                                                 const uint64_t* twi, uint64_t q, uint64_t inv1, uint64_t* dst) {
  typedef IPRounds<LOGB, W> G;
  constexpr bool LAST = POS + G::RW >= LOGB;
  constexpr int R = LAST ? LOGB - POS : G::RW;
#pragma unroll
  for (int k = 0; k < (W >> R); ++k) {
    int c, b;
    ip_item<R, LOGB, W>(k, POS, c, b);
    uint64_t y[1 << R];
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) y[i] = lds[ip_lds<LOGB>(b + (i << POS), c)];
    const uint32_t blk = tile * G::KC + c;
    round_regs<R, true, AR, false, false, POS>(y, b, POS, (int)(blk & 15), LOGB, blk >> 4, s0, log_n, twi, q);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      if constexpr (LAST) at_u32(dst, ip_word<LOGB, W>(tile, b + (i << POS), c)) = inv_row_out<AR>(y[i], q, inv1);
      else lds[ip_lds<LOGB>(b + (i << POS), c)] = y[i];
    }
  }
  if constexpr (!LAST) {
    wave_lds_wait();
    ip_inv_rounds_up<LOGB, AR, W, POS + R>(lds, tile, log_n, s0, twi, q, inv1, dst);
  }
}
template <int LOGB, int AR, int W>
__device__ __forceinline__ void ip_inverse_row_store(uint64_t (&x)[W], uint64_t* lds, uint32_t tile, int log_n,
                                                     const uint64_t* twi, uint64_t q, uint64_t inv1, uint64_t* dst) {
  typedef IPRounds<LOGB, W> G;
  const uint32_t s0 = (uint32_t)logb_col(log_n);
  int col, base;
  ip_item<G::RW, LOGB, W>(0, 0, col, base);
  {
    const uint32_t blk = tile * G::KC + col;
    round_regs<G::RW, true, AR, false, false, 0>(x, base, 0, (int)(blk & 15), LOGB, blk >> 4, s0, log_n, twi, q);
  }
  wave_lds_wait();  // the wave has read its columns' previous contents
#pragma unroll
  for (int i = 0; i < W; ++i) lds[ip_lds<LOGB>(base + i, col)] = x[i];
  wave_lds_wait();
  ip_inv_rounds_up<LOGB, AR, W, G::RW>(lds, tile, log_n, s0, twi, q, inv1, dst);
}

// acc: item b at acc + b*acc_bstride, [2][K][N] (special limbs only).
template <int LOGB, int LOGN, int W = 8>
__global__ __launch_bounds__((IPRounds<LOGB, W>::THREADS)) __attribute__((amdgpu_waves_per_eu(W == 8 ? 2 : (LOGN ? 4 : 3)))) void ip_special_kernel(
    RowIPArgs a, const uint64_t* twi) {
  __shared__ uint64_t lds[(1 << LOGB) * IPRounds<LOGB, W>::KC];
  __shared__ ulonglong2 twl[IPRounds<LOGB, W>::KC * ((1 << LOGB) - 1)];
  const GridPos g0 = a.shared_key ? row_grid_pos<true>() : row_grid_pos<false>();
  const int t = g0.job + a.t0;  // a special limb
  const int keyl = a.L + (t - a.level - 1);
  const PrimeConst& pc = a.prime[keyl];
  const int log_n = LOGN ? LOGN : a.log_n;
  const uint32_t s0 = (uint32_t)logb_col(log_n);
  const uint64_t* tw_i = twi + ((uint64_t)keyl << (log_n + 1));
  ip_stage_twiddles<LOGB, W>(twl, a.tw + ((uint64_t)keyl << (log_n + 1)), g0.tile, s0);
  __syncthreads();  // every wave reads the twiddles every thread staged
  for (int k = 0; k < a.items_per_wg; ++k) {
    GridPos gp = g0;
    gp.item = g0.item * a.items_per_wg + k;
    if (gp.item >= a.n_items) break;
    uint64_t accb[W], acca[W];
    const int far = fwd_ar(pc.q);
    if (far == AR_LAZY)
      ip_accumulate<LOGB, LOGN, AR_LAZY, W>(a, lds, twl, pc, keyl, gp, accb, acca);
    else if (far == AR_HARVEY)
      ip_accumulate<LOGB, LOGN, AR_HARVEY, W>(a, lds, twl, pc, keyl, gp, accb, acca);
    else
      ip_accumulate<LOGB, LOGN, AR_STRICT, W>(a, lds, twl, pc, keyl, gp, accb, acca);
    // remove the 2^-64: [0, 4q), the range the lazy and Harvey inverse
    // butterflies take; the exact-quotient ones take [0, 2q)
    const int iar = inv_ar(pc.q);
#pragma unroll
    for (int i = 0; i < W; ++i) {
      accb[i] = mul_shoup_lazy(accb[i], pc.r64, pc.r64p, pc.q);
      acca[i] = mul_shoup_lazy(acca[i], pc.r64, pc.r64p, pc.q);
    }
    if (iar == AR_STRICT) {
      const uint64_t two_q = 2 * pc.q;
#pragma unroll
      for (int i = 0; i < W; ++i) {
        accb[i] = accb[i] >= two_q ? accb[i] - two_q : accb[i];
        acca[i] = acca[i] >= two_q ? acca[i] - two_q : acca[i];
      }
    }
    uint64_t* ob = a.acc + gp.item * a.acc_bstride + ((uint64_t)(t - a.level - 1) << log_n);
    uint64_t* oa = ob + ((uint64_t)a.K << log_n);
    if (iar == AR_LAZY) {
      ip_inverse_row_store<LOGB, AR_LAZY, W>(accb, lds, gp.tile, log_n, tw_i, pc.q, pc.inv1, ob);
      ip_inverse_row_store<LOGB, AR_LAZY, W>(acca, lds, gp.tile, log_n, tw_i, pc.q, pc.inv1, oa);
    } else if (iar == AR_HARVEY) {
      ip_inverse_row_store<LOGB, AR_HARVEY, W>(accb, lds, gp.tile, log_n, tw_i, pc.q, pc.inv1, ob);
      ip_inverse_row_store<LOGB, AR_HARVEY, W>(acca, lds, gp.tile, log_n, tw_i, pc.q, pc.inv1, oa);
    } else {
      ip_inverse_row_store<LOGB, AR_STRICT, W>(accb, lds, gp.tile, log_n, tw_i, pc.q, pc.inv1, ob);
      ip_inverse_row_store<LOGB, AR_STRICT, W>(acca, lds, gp.tile, log_n, tw_i, pc.q, pc.inv1, oa);
    }
  }
}

typedef void (*IPSpecialFn)(RowIPArgs, const uint64_t*);

// Words per thread of the special-limb inner product (IPRounds): 8 measured
// faster than 4 here (the extra inverse round and its twiddle loads cost more
// than the added waves gain).
constexpr int kSpecialW = 8;

IPSpecialFn pick_ip_special(int log_n, int logb) {
  if (log_n == 16 && logb == 8) return ip_special_kernel<8, 16, kSpecialW>;
  switch (logb) {
    case 5: return ip_special_kernel<5, 0, kSpecialW>;
    case 6: return ip_special_kernel<6, 0, kSpecialW>;
    case 7: return ip_special_kernel<7, 0, kSpecialW>;
    case 8: return ip_special_kernel<8, 0, kSpecialW>;
  }
  return nullptr;
}

// ---------------------------------------------------------------------------
// Inner product of the ciphertext limbs fused with the final combination:
// per (tile, limb i <= l, item) the workgroup accumulates the key inner
// product in registers (as ip_accumulate), then runs the forward row pass of
// the ModDown output w of both components on the same tile, and stores
//   out_c[i] = acc_c * P^-1 - NTT(w_c) (+ add_c) (+ accum_c)
// directly: the ciphertext-limb accumulators never go to memory.  The
// factors 2^64 (Montgomery) and P^-1 are one Shoup multiplication by
// [2^64 P^-1]_{q_i}.
struct CombIPArgs {
  RowIPArgs ip;
  const uint64_t* W;  // item b: W + b*W_bstride, [2][nq][N] (forward column pass done)
  uint64_t W_bstride;
  const uint64_t* add[2];  // component c's additive term, item b at + b*add_bstride, [nq][N]
  uint64_t add_bstride;
  uint32_t add_g[kMaxChunk];  // item b's add terms are read through tau_g (0: as they are)
  const uint64_t* accum;      // [2][nq][N] per item, or NULL
  uint64_t accum_bstride;
  uint64_t* out;
  uint64_t out_bstride;
  int out_comp_limbs;
  const uint64_t* pinv64;  // [L][2]: {[2^64 P^-1]_{q_i}, Shoup}
};

template <int LOGB, int LOGN, int AR, int W>
__device__ __forceinline__ void comb_ip_body(const CombIPArgs& a, uint64_t* lds, const ulonglong2* twl,
                                             const PrimeConst& pc, int i, const GridPos& gp) {
  constexpr int H = W / 2;
  const int log_n = LOGN ? LOGN : a.ip.log_n;
  const int item = gp.item;
  const uint64_t q = pc.q;
  uint64_t acc[2][W];
  ip_accumulate<LOGB, LOGN, AR, W>(a.ip, lds, twl, pc, i, gp, acc[0], acc[1]);
  const uint64_t cw = a.pinv64[2 * i], cwp = a.pinv64[2 * i + 1];
  // Lazy primes in (2^33, 2^56): the row pass leaves NTT(w) below 65q < 2^63,
  // which reduce_hi takes to [0, 2q); with acc*P^-1 in [0, 4q) and canonical
  // add and accum terms, acc + 2q - w + add + accum lies below 8q and is
  // reduced once.  Otherwise every term is made canonical first.
  const bool fast = AR == AR_LAZY && q > kReduceHiMin && q < (1ull << 56);
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < W; ++r) {
      acc[c][r] = mul_shoup_lazy(acc[c][r], cw, cwp, q);
      if (!fast) acc[c][r] = reduce_4q(acc[c][r], q);
    }
  int col, base;
  ip_item<IPRounds<LOGB, W>::RW, LOGB, W>(0, 0, col, base);
  const uint32_t w0 = ip_word<LOGB, W>(gp.tile, base, col);
  const uint32_t ag = a.add_g[item];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    // the additive terms load during the row pass's later rounds
    ip_row_pass_first<LOGB, AR, W>(a.W + item * a.W_bstride + ((uint64_t)(c * a.ip.level + c + i) << log_n), lds,
                                   twl, gp.tile, log_n, q);
    uint64_t add[W], accum[W];
#pragma unroll
    for (int r = 0; r < W; ++r) add[r] = accum[r] = 0;
    if (a.add[c]) {
      const uint64_t* ad = a.add[c] + item * a.add_bstride + ((uint64_t)i << log_n);
#pragma unroll
      for (int r = 0; r < W; ++r) add[r] = at_u32(ad, ag ? automorph_src(w0 + r, ag, log_n) : w0 + r);
    }
    if (a.accum) {
      const ulonglong2* ac =
          reinterpret_cast<const ulonglong2*>(a.accum + item * a.accum_bstride + ((uint64_t)(c * (a.ip.level + 1) + i) << log_n));
#pragma unroll
      for (int r = 0; r < H; ++r) {
        const ulonglong2 v = at_u32(ac, (w0 >> 1) + r);
        accum[2 * r] = v.x;
        accum[2 * r + 1] = v.y;
      }
    }
    uint64_t x[W];
    ip_row_pass_rest<LOGB, AR, W>(x, lds, twl, gp.tile, log_n, q);
    ulonglong2* o = reinterpret_cast<ulonglong2*>(a.out + item * a.out_bstride +
                                                  ((uint64_t)(c * a.out_comp_limbs + i) << log_n));
    if (fast) {
      const uint64_t two_q = 2 * q, four_q = 4 * q;
      const uint32_t m = (uint32_t)pc.inv1;
#pragma unroll
      for (int r = 0; r < H; ++r) {
        uint64_t e0 = acc[c][2 * r] + two_q - reduce_hi(x[2 * r], q, m) + add[2 * r] + accum[2 * r];
        uint64_t e1 = acc[c][2 * r + 1] + two_q - reduce_hi(x[2 * r + 1], q, m) + add[2 * r + 1] + accum[2 * r + 1];
        e0 = reduce_4q(e0 >= four_q ? e0 - four_q : e0, q);
        e1 = reduce_4q(e1 >= four_q ? e1 - four_q : e1, q);
        at_u32(o, (w0 >> 1) + r) = make_ulonglong2(e0, e1);
      }
    } else {
#pragma unroll
      for (int r = 0; r < H; ++r) {
        ulonglong2 v;
        uint64_t e0 = sub_mod(acc[c][2 * r], reduce64(x[2 * r], q, pc.inv1), q);
        uint64_t e1 = sub_mod(acc[c][2 * r + 1], reduce64(x[2 * r + 1], q, pc.inv1), q);
        v.x = add_mod(add_mod(e0, add[2 * r], q), accum[2 * r], q);
        v.y = add_mod(add_mod(e1, add[2 * r + 1], q), accum[2 * r + 1], q);
        at_u32(o, (w0 >> 1) + r) = v;
      }
    }
  }
}

template <int LOGB, int LOGN, int W = 8>
__global__ __launch_bounds__((IPRounds<LOGB, W>::THREADS)) __attribute__((amdgpu_waves_per_eu(W == 8 ? 2 : (LOGN ? 4 : 3)))) void comb_ip_kernel(
    CombIPArgs a) {
  __shared__ uint64_t lds[(1 << LOGB) * IPRounds<LOGB, W>::KC];
  __shared__ ulonglong2 twl[IPRounds<LOGB, W>::KC * ((1 << LOGB) - 1)];
  const GridPos g0 = a.ip.shared_key ? row_grid_pos<true>() : row_grid_pos<false>();
  const int i = g0.job;  // a ciphertext limb
  const PrimeConst& pc = a.ip.prime[i];
  const int log_n = LOGN ? LOGN : a.ip.log_n;
  ip_stage_twiddles<LOGB, W>(twl, a.ip.tw + ((uint64_t)i << (log_n + 1)), g0.tile, (uint32_t)logb_col(log_n));
  __syncthreads();  // every wave reads the twiddles every thread staged
  for (int k = 0; k < a.ip.items_per_wg; ++k) {
    GridPos gp = g0;
    gp.item = g0.item * a.ip.items_per_wg + k;
    if (gp.item >= a.ip.n_items) break;
    const int far = fwd_ar(pc.q);
    if (far == AR_LAZY)
      comb_ip_body<LOGB, LOGN, AR_LAZY, W>(a, lds, twl, pc, i, gp);
    else if (far == AR_HARVEY)
      comb_ip_body<LOGB, LOGN, AR_HARVEY, W>(a, lds, twl, pc, i, gp);
    else
      comb_ip_body<LOGB, LOGN, AR_STRICT, W>(a, lds, twl, pc, i, gp);
  }
}

typedef void (*CombIPFn)(CombIPArgs);

// Words per thread of the combining kernel (IPRounds): 4, at 4 waves per
// SIMD for N = 2^16, measured faster than 8 at 2 waves.
constexpr int kCombW = 4;

CombIPFn pick_comb_ip(int log_n, int logb) {
  if (log_n == 16 && logb == 8) return comb_ip_kernel<8, 16, kCombW>;
  switch (logb) {
    case 5: return comb_ip_kernel<5, 0, kCombW>;
    case 6: return comb_ip_kernel<6, 0, kCombW>;
    case 7: return comb_ip_kernel<7, 0, kCombW>;
    case 8: return comb_ip_kernel<8, 0, kCombW>;
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
// automorphism.  Lazy Montgomery products as in ip_accumulate.
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
  const int fold = mont_fold(q);
  int since = 0;
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
    if (++since == fold) {  // mont_fold(m) products since the last reduction
      since = 0;
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

// ModUp of the inverse-row-passed input Y (item b at Y + b*ystride,
// [nq][N]): the inverse column pass times [qhat_i^-1 N^-1] (canonical y_i), the
// conversion to every target limb of every digit, and the forward column
// pass of the converted limbs, into E (item b at E + b*estride,
// [beta][next][N], lazy).  Y is overwritten.
// Debug dumps of the key switch's intermediates, for localising a mismatch
// against the oracle to one stage.  When the environment variable
// CKKS_DEBUG_DUMP names a directory, each chunk of a key switch gets the next
// sequence number and, after the step that produces it, every item's buffer
// is copied to the host and written as raw little-endian 64-bit words to
// <dir>/ks<seq>_<stage>_item<k>.u64:
//   modup_in     [l+1][N]     y_i = [x_i qhat_i^-1]_{q_i}, coefficient form
//   modup_out    [beta][next][N]  the ModUp conversion, coefficient form,
//                congruent to the exact value (below 6q); the slots of a
//                digit's own limbs are not written
//   moddown_in   [2][K][N]    y_k = [acc_k phat_k^-1]_{p_k}, coefficient form
//   moddown_out  [2][l+1][N]  the ModDown conversion times P^-1, coefficient
//                form, congruent (below 6q)
// The stream is synchronised for every dump.  Allocation-free calls dump
// nothing.
static std::atomic<int> g_dump_seq{0};

int debug_dump(Ctx* c, hipStream_t s, const char* stage, int n_items, const uint64_t* base, uint64_t stride,
               uint64_t words) {
  const char* dir = getenv("CKKS_DEBUG_DUMP");
  if (!dir || !*dir || c->no_alloc || c->dump_seq < 0) return CKKS_OK;
  CKKS_HIP_CHECK(hipStreamSynchronize(s));
  std::vector<uint64_t> h(words);
  for (int k = 0; k < n_items; ++k) {
    CKKS_HIP_CHECK(hipMemcpy(h.data(), base + k * stride, words * 8, hipMemcpyDeviceToHost));
    char name[64];
    snprintf(name, sizeof(name), "/ks%06d_%s_item%d.u64", c->dump_seq, stage, k);
    const std::string path = std::string(dir) + name;
    FILE* f = fopen(path.c_str(), "wb");
    if (!f) return set_error(CKKS_EINVAL, "CKKS_DEBUG_DUMP: cannot write " + path);
    const size_t wrote = fwrite(h.data(), 8, words, f);
    fclose(f);
    if (wrote != words) return set_error(CKKS_EINVAL, "CKKS_DEBUG_DUMP: short write to " + path);
  }
  return CKKS_OK;
}

int modup_steps(Ctx* c, hipStream_t s, int level, int n_items, uint64_t* Y, uint64_t ystride, uint64_t* E,
                uint64_t estride) {
  const int nq = level + 1, next = nq + (int)c->K, beta = c->beta(level);
  int rc;
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
    if ((rc = ntt_pass_only(c, s, Y, Y, ystride, ystride, n_items, jobs, true, false, 2, c->d_modup, off))) return rc;
  }
  if ((rc = debug_dump(c, s, "modup_in", n_items, Y, ystride, (uint64_t)nq * c->N))) return rc;
  ModUpArgs mu;
  memset(&mu, 0, sizeof(mu));
  mu.x = Y;
  mu.out = E;
  mu.x_bstride = ystride;
  mu.out_bstride = estride;
  mu.tables = c->d_modup;
  mu.prime = c->d_prime;
  mu.n = c->N;
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
  if ((rc = debug_dump(c, s, "modup_out", n_items, E, estride, (uint64_t)beta * next * c->N))) return rc;
  NttJobs jobs;
  for (int j = 0; j < beta; ++j)
    for (int t = 0; t < next; ++t) {
      if (t >= c->modup[level][j].lo && t < c->modup[level][j].hi) continue;
      jobs.add(j * next + t, j * next + t, c->ext_prime(level, t));
    }
  return ntt_pass_only(c, s, E, E, estride, estride, n_items, jobs, false, true, 0, nullptr, nullptr);
}

// ModDown of the special accumulators A (item b at A + b*astride, [2][K][N],
// inverse row pass done): the inverse column pass times [phat_k^-1 N^-1]
// (y_k, canonical), the centred conversion to the ciphertext limbs (times
// P^-1), and their forward column pass, into W (item b at W + b*wstride,
// [2][nq][N], lazy).  A is overwritten.
int moddown_steps(Ctx* c, hipStream_t s, int level, int n_items, uint64_t* A, uint64_t astride, uint64_t* W,
                  uint64_t wstride) {
  const int nq = level + 1, K = (int)c->K;
  int rc;
  {
    NttJobs jobs;
    uint32_t off[kMaxJobs];
    for (int comp = 0; comp < 2; ++comp)
      for (int k = 0; k < K; ++k) {
        off[jobs.n] = (uint32_t)(c->md.phinv + 2 * k);
        jobs.add(comp * K + k, comp * K + k, (int)c->L + k);
      }
    if ((rc = ntt_pass_only(c, s, A, A, astride, astride, n_items, jobs, true, false, 2, c->d_moddown, off))) return rc;
  }
  if ((rc = debug_dump(c, s, "moddown_in", n_items, A, astride, 2ull * K * c->N))) return rc;
  ModDownArgs md;
  memset(&md, 0, sizeof(md));
  md.acc = A;
  md.w = W;
  md.acc_bstride = astride;
  md.w_bstride = wstride;
  md.conv = c->d_moddown + c->md.conv;
  md.prime = c->d_prime;
  md.n = c->N;
  md.level = level;
  md.acc_comp_limbs = K;
  md.acc_k0 = 0;
  md.L = (int)c->L;
  md.K = K;
  if ((rc = launch_moddown_conv(c, s, md, n_items))) return rc;
  if ((rc = debug_dump(c, s, "moddown_out", n_items, W, wstride, 2ull * nq * c->N))) return rc;
  NttJobs jobs;
  for (int comp = 0; comp < 2; ++comp)
    for (int i = 0; i < nq; ++i) jobs.add(comp * nq + i, comp * nq + i, i);
  return ntt_pass_only(c, s, W, W, wstride, wstride, n_items, jobs, false, true, 0, nullptr, nullptr);
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
    md.acc_comp_limbs = next;
    md.acc_k0 = nq;
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

// Workspace of the fused pipeline per item: Y [nq] (inverse row pass of the
// input), E [beta][next] (raised digits after the forward column pass), A
// [2][K] (special accumulators after the inverse row pass), W [2][nq]
// (ModDown output after the forward column pass).
size_t fused_ws_words(const Ctx* c, int level) {
  const size_t n = c->N, nq = level + 1, next = nq + c->K, beta = c->beta(level);
  return n * (nq + beta * next + 2 * (size_t)c->K + 2 * nq);
}

size_t ks_ws_words(const Ctx* c, int level) { return fused_ws_words(c, level); }

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
    if ((rc = launch_gather(c, s, ga, nq, n_in))) return rc;
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

// The fused pipeline (digits and special primes of at most 8 limbs):
//   intt_row_gather   inverse row pass of tau_g(c1)                 -> Y
//   modup pass        inverse column pass of each digit, ModUp,
//                     forward column pass of every target limb      -> E
//   ip_special        forward row pass + inner product of the K
//                     special limbs, inverse row pass               -> A
//   moddown pass      inverse column pass of A, centred ModDown,
//                     forward column pass of every ciphertext limb  -> W
//   comb_ip           forward row pass + inner product of the
//                     ciphertext limbs, forward row pass of W,
//                     acc*P^-1 - NTT(w) (+ add) (+ accum)           -> out
int ks_chunk_fused(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, uint64_t d_stride,
                   uint64_t add_stride, uint64_t accum_stride, uint64_t out_stride, int out_comp_limbs, uint64_t* ws) {
  const uint32_t N = c->N;
  const int log_n = (int)c->log_n;
  const int nq = level + 1, next = nq + (int)c->K, beta = c->beta(level), K = (int)c->K;
  const uint64_t per = fused_ws_words(c, level);
  uint64_t* Y = ws;
  uint64_t* E = Y + (uint64_t)nq * N;
  uint64_t* A = E + (uint64_t)beta * next * N;
  uint64_t* W = A + (uint64_t)2 * K * N;
  const int lr = logb_row(log_n);
  int rc;
  {
    const char* dump = getenv("CKKS_DEBUG_DUMP");
    c->dump_seq = (dump && *dump) ? g_dump_seq++ : -1;
  }
  {
    GatherArgs ga;
    memset(&ga, 0, sizeof(ga));
    ga.src = it[0].d;
    ga.src_bstride = d_stride;
    ga.dst = Y;
    ga.dst_bstride = per;
    ga.tw = c->d_tw_inv;
    ga.prime = c->d_prime;
    for (int i = 0; i < n_items; ++i) ga.g[i] = it[i].g;
    ga.log_n = log_n;
    if ((rc = launch_gather(c, s, ga, nq, n_items))) return rc;
  }
  if ((rc = modup_steps(c, s, level, n_items, Y, per, E, per))) return rc;
  RowIPArgs ip;
  memset(&ip, 0, sizeof(ip));
  ip.E = E;
  ip.E_bstride = per;
  ip.T = it[0].d;
  ip.T_bstride = d_stride;
  for (int i = 0; i < n_items; ++i) ip.g[i] = it[i].g;
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
  ip.K = K;
  ip.n_items = n_items;
  {
    RowIPArgs sp = ip;
    sp.acc = A;
    sp.acc_bstride = per;
    sp.t0 = nq;
    sp.items_per_wg = 2;
    IPSpecialFn fn = pick_ip_special(log_n, lr);
    if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
    const double units = (double)K * ((double)beta * (N / 2) * lr + N * (2.0 * beta + 2) + 2.0 * (N / 2) * lr);
    TraceScope ts(c, s, "ip_special", units * n_items);
    const int logkc = ip_logkc(lr, kSpecialW);
    hipLaunchKernelGGL(fn, dim3(N >> (lr + logkc), K, (n_items + 1) / 2), dim3((1u << (lr + logkc)) / kSpecialW), 0, s,
                       sp, c->d_tw_inv);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  if ((rc = moddown_steps(c, s, level, n_items, A, per, W, per))) return rc;
  {
    CombIPArgs ca;
    memset(&ca, 0, sizeof(ca));
    ca.ip = ip;
    ca.ip.t0 = 0;
    ca.ip.items_per_wg = 2;
    ca.W = W;
    ca.W_bstride = per;
    ca.add[0] = it[0].add[0];
    ca.add[1] = it[0].add[1];
    ca.add_bstride = add_stride;
    for (int i = 0; i < n_items; ++i) ca.add_g[i] = it[i].add_g;
    ca.accum = it[0].accum;
    ca.accum_bstride = accum_stride;
    ca.out = it[0].out;
    ca.out_bstride = out_stride;
    ca.out_comp_limbs = out_comp_limbs;
    ca.pinv64 = c->d_moddown + c->md.pinv64;
    CombIPFn fn = pick_comb_ip(log_n, lr);
    if (!fn) return set_error(CKKS_EINTERNAL, "unsupported NTT pass size");
    double units = 0;
    for (int j = 0; j < beta; ++j) {
      const int na = c->modup[level][j].hi - c->modup[level][j].lo;
      units += (double)(nq - na) * (N / 2) * lr;  // row passes of the converted ciphertext limbs
    }
    units += (double)nq * (N * (2.0 * beta + 2) + 2.0 * ((N / 2) * lr + N));
    TraceScope ts(c, s, "comb_ip", units * n_items);
    const int logkc = ip_logkc(lr, kCombW);
    hipLaunchKernelGGL(fn, dim3(N >> (lr + logkc), nq, (n_items + 1) / 2), dim3((1u << (lr + logkc)) / kCombW), 0,
                       s, ca);
    CKKS_HIP_CHECK(hipGetLastError());
  }
  return CKKS_OK;
}

int ks_chunk(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, uint64_t d_stride,
             uint64_t add_stride, uint64_t accum_stride, uint64_t out_stride, int out_comp_limbs, uint64_t* ws) {
  return ks_chunk_fused(c, s, level, n_items, it, d_stride, add_stride, accum_stride, out_stride, out_comp_limbs, ws);
}

}  // namespace ckks
