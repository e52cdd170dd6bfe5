// Row passes with the tile's twiddles staged in LDS, for kernels that run the
// row pass of several limbs or items on one tile: the key-switch inner
// products (a forward row pass per digit), the batched inverse NTT's row pass
// and the key switch's first inverse pass of c1 (one per item of the
// workgroup).  The twiddles a tile of KC columns needs, KC * (2^LOGB - 1)
// Shoup pairs, are read from the table once per workgroup instead of once per
// butterfly group and item.  Every wave works on its own columns of the tile
// in every round (ip_item), so only the twiddle staging needs a workgroup
// barrier.
#pragma once
#include "automorph.h"
#include "ntt_core.h"

namespace ckks {
namespace nttc {

// A workgroup's tile is KC columns of 2^LOGB rows.  Every thread holds W
// words (8, or 4 for more waves per SIMD at half the registers) in every
// register round and ends the forward pass with W consecutive words of one
// column: the layout the multiply phase reads the key digits in.  The LOGB
// stages run as rounds of log2(W) stages, the first round taking what is
// left (W = 8 at 2^8 rows: 2, 3, 3; W = 4: 2, 2, 2, 2).  KC is 8 (W = 8) or 4
// (W = 4) from 2^7 rows on, twice that below, so that several workgroups
// share a CU.
__host__ __device__ constexpr int ip_logkc(int logb, int w = 8) { return (logb >= 7 ? 3 : 4) - (w == 4 ? 1 : 0); }

template <int LOGB, int W = 8>
struct IPRounds {
  static_assert(W == 8 || W == 4, "words per thread");
  static constexpr int RW = W == 8 ? 3 : 2;                    // stages per full round
  static constexpr int NR = (LOGB + RW - 1) / RW;              // rounds
  static constexpr int R0 = LOGB - RW * (NR - 1);              // stages of the first round
  static constexpr int R3 = 3;                                 // W = 8 names: the last round,
  static constexpr int R2 = LOGB >= 6 ? 3 : LOGB - 3;          // the one before it,
  static constexpr int R1 = LOGB - R2 - R3;                    // the first (0 when two suffice)
  static constexpr int LOGKC = ip_logkc(LOGB, W);
  static constexpr int KC = 1 << LOGKC;
  static constexpr int THREADS = (KC << LOGB) / W;
  static constexpr int CPW = (64 * W) >> LOGB;                 // columns per wave
};

// Work item k (k < W >> R) of the calling thread in a register round of R
// stages at row bit pos.  Wave w takes the items of its own CPW columns
// (KC columns over THREADS / 64 waves), consecutive lanes taking consecutive
// items; for R = log2(W) this is the thread's column in every other round
// too, so each wave touches only its own columns of the LDS tile in every
// round of a pass, and the rounds need no workgroup barrier.
template <int R, int LOGB, int W = 8>
__device__ __forceinline__ void ip_item(int k, int pos, int& col, int& base) {
  constexpr int NB = 1 << (LOGB - R);  // items per column
  const int u = k * 64 + ((int)threadIdx.x & 63);
  col = ((int)threadIdx.x >> 6) * IPRounds<LOGB, W>::CPW + u / NB;
  const int b = u % NB;
  base = ((b >> pos) << (pos + R)) | (b & ((1 << pos) - 1));
}

// global word index (within the limb) of tile element (row, col)
template <int LOGB, int W = 8>
__device__ __forceinline__ uint32_t ip_word(uint32_t tile, int row, int col) {
  return ((tile * IPRounds<LOGB, W>::KC + col) << LOGB) + row;
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
template <int LOGB, int W = 8>
__device__ __forceinline__ void ip_stage_twiddles(ulonglong2* twl, const uint64_t* tw, uint32_t tile, uint32_t s0) {
  typedef IPRounds<LOGB, W> G;
  constexpr int ENTRIES = G::KC * ((1 << LOGB) - 1);
  for (int e = threadIdx.x; e < ENTRIES; e += G::THREADS) {
    const int d = 31 - __clz((e >> G::LOGKC) + 1);
    const uint32_t g = (1u << (s0 + d)) + (tile << (G::LOGKC + d)) + (uint32_t)(e - G::KC * ((1 << d) - 1));
    twl[e] = *reinterpret_cast<const ulonglong2*>(tw + 2 * (uint64_t)g);
  }
}

// R forward stages on the 2^R words of one item (rows base + (i << pos) of
// column col), twiddles from the LDS copy.
template <int R, int LOGB, int AR, int W = 8>
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
      const ulonglong2 w = twl[IPRounds<LOGB, W>::KC * ((1 << d) - 1) + (col << d) + (row >> (LOGB - d))];
#pragma unroll
      for (int m = 0; m < half; ++m) ct_butterfly<AR>(x[i0 + m], x[i0 + m + half], w.x, w.y, q);
    }
  }
}

// One register round of R forward stages on row bits [POS, POS+R): item k of
// the thread (k < W >> R, ip_item); its words are rows base + (i << POS) of
// column col, read from global memory (src) or LDS and left in LDS or in x[].
template <int R, int POS, int LOGB, int AR, bool FROM_GLOBAL, bool TO_LDS, int W = 8>
__device__ __forceinline__ void ip_round(uint64_t (&x)[W], const uint64_t* src, uint64_t* lds, const ulonglong2* twl,
                                         uint32_t tile, int log_n, uint64_t q) {
  constexpr int NI = W >> R;
  uint64_t y[NI][1 << R];
  int col[NI], base[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    ip_item<R, LOGB, W>(k, POS, col[k], base[k]);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      const int row = base[k] + (i << POS);
      y[k][i] = FROM_GLOBAL ? at_u32(src, ip_word<LOGB, W>(tile, row, col[k])) : lds[ip_lds<LOGB>(row, col[k])];
    }
  }
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    ip_butterflies<R, LOGB, AR, W>(y[k], base[k], POS, col[k], twl, q);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      if (TO_LDS) lds[ip_lds<LOGB>(base[k] + (i << POS), col[k])] = y[k][i];
      else x[(k << R) + i] = y[k][i];
    }
  }
}

// Forward row pass of one limb (src, lazy column-pass output) on the tile,
// in two calls: ip_row_pass_first reads the limb and runs the first register
// round into the LDS tile; ip_row_pass_rest runs the other rounds and leaves
// the thread rows base..base+7 of its column in x[] (lazy).  Loads issued
// between the two calls (the key words of the inner product) are in flight
// during the other rounds without holding up the first round's wait for its
// own loads.
template <int LOGB, int AR, int W = 8>
__device__ __forceinline__ void ip_row_pass_first(const uint64_t* src, uint64_t* lds, const ulonglong2* twl,
                                                  uint32_t tile, int log_n, uint64_t q) {
  typedef IPRounds<LOGB, W> G;
  uint64_t unused[W];
  wave_lds_wait();  // the wave has read its columns' previous contents
  ip_round<G::R0, LOGB - G::R0, LOGB, AR, true, true, W>(unused, src, lds, twl, tile, log_n, q);
}
// The rounds below row bit POS, through the LDS tile, the last into x[].
template <int LOGB, int AR, int W, int POS>
__device__ __forceinline__ void ip_rounds_down(uint64_t (&x)[W], uint64_t* lds, const ulonglong2* twl, uint32_t tile,
                                               int log_n, uint64_t q) {
  constexpr int RW = IPRounds<LOGB, W>::RW;
  constexpr int P = POS - RW;
  wave_lds_wait();
  if constexpr (P > 0) {
    ip_round<RW, P, LOGB, AR, false, true, W>(x, nullptr, lds, twl, tile, log_n, q);
    ip_rounds_down<LOGB, AR, W, P>(x, lds, twl, tile, log_n, q);
  } else {
    ip_round<RW, 0, LOGB, AR, false, false, W>(x, nullptr, lds, twl, tile, log_n, q);
  }
}
template <int LOGB, int AR, int W = 8>
__device__ __forceinline__ void ip_row_pass_rest(uint64_t (&x)[W], uint64_t* lds, const ulonglong2* twl,
                                                 uint32_t tile, int log_n, uint64_t q) {
  ip_rounds_down<LOGB, AR, W, LOGB - IPRounds<LOGB, W>::R0>(x, lds, twl, tile, log_n, q);
}

// R inverse (Gentleman-Sande) stages on the 2^R words of one item (rows
// base + (i << pos) of column col), highest stage first, twiddles from the
// LDS copy of the inverse table.  KDONE: stages of this pass already done
// (the bound of the lazy butterflies).
template <int R, int LOGB, int AR, int KDONE, int W = 8>
__device__ __forceinline__ void ip_inv_butterflies(uint64_t (&x)[1 << R], int base, int pos, int col,
                                                   const ulonglong2* twl, uint64_t q) {
  constexpr int E = 1 << R;
#pragma unroll
  for (int ss = 0; ss < R; ++ss) {
    const int s = R - 1 - ss;
    const int half = E >> (s + 1);
    const int d = LOGB - pos - R + s;
#pragma unroll
    for (int g = 0; g < (1 << s); ++g) {
      const int i0 = g * 2 * half;
      const int row = base + (i0 << pos);
      const ulonglong2 w = twl[IPRounds<LOGB, W>::KC * ((1 << d) - 1) + (col << d) + (row >> (LOGB - d))];
#pragma unroll
      for (int m = 0; m < half; ++m)
        gs_butterfly_ar<AR>(x[i0 + m], x[i0 + m + half], w.x, w.y, q, (4 * q) << (KDONE + ss));
    }
  }
}

// Output word of an inverse row pass, for the inverse column pass that
// follows (it takes words below 4q): the lazy butterflies end below 2^10 q and
// are reduced once, to [0, 2.5q) (reduce_hi) or [0, q); the other ranges are
// already below 4q.
template <int AR>
__device__ __forceinline__ uint64_t inv_row_out(uint64_t v, uint64_t q, uint64_t inv1) {
  if (AR != AR_LAZY) return v;
  return q > kReduceHiMin ? reduce_hi(v, q, (uint32_t)inv1) : reduce64(v, q, inv1);
}

// The inverse row pass's rounds from row bit POS up, through the LDS tile
// (rounds of log2(W) stages, the last taking what is left); the last round
// stores the pass's output to dst.
template <int LOGB, int AR, int W, int POS>
__device__ __forceinline__ void ip_inv_rounds_up(uint64_t* dst, uint64_t* lds, const ulonglong2* twl, uint32_t tile,
                                                 uint64_t q, uint64_t inv1) {
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
    ip_inv_butterflies<R, LOGB, AR, POS, W>(y, b, POS, c, twl, q);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      if constexpr (LAST) at_u32(dst, ip_word<LOGB, W>(tile, b + (i << POS), c)) = inv_row_out<AR>(y[i], q, inv1);
      else lds[ip_lds<LOGB>(b + (i << POS), c)] = y[i];
    }
  }
  if constexpr (!LAST) {
    wave_lds_wait();
    ip_inv_rounds_up<LOGB, AR, W, POS + R>(dst, lds, twl, tile, q, inv1);
  }
}

// Inverse row pass of one limb on the tile: src holds canonical (or below
// 4q) words, dst receives the pass's output for the column pass that follows
// (below 4q: inv_row_out); with g nonzero the input is read through tau_g.
// The first round takes the thread's W consecutive words (16-byte loads, or
// word by word through tau_g) on the low row bits in registers; the other
// rounds go up through the LDS tile, and the last one's stores cover
// consecutive rows across the wave.
template <int LOGB, int AR, int W = 8>
__device__ __forceinline__ void ip_inv_row_pass(const uint64_t* src, uint64_t* dst, uint64_t* lds,
                                                const ulonglong2* twl, uint32_t tile, uint64_t q, uint64_t inv1,
                                                uint32_t g = 0, int log_n = 0) {
  typedef IPRounds<LOGB, W> G;
  int col, base;
  ip_item<G::RW, LOGB, W>(0, 0, col, base);
  uint64_t x[W];
  const uint32_t w0 = ip_word<LOGB, W>(tile, base, col);
  if (g) {  // the input through tau_g (automorph.h): word j comes from word automorph_src(j, g)
#pragma unroll
    for (int i = 0; i < W; ++i) x[i] = at_u32(src, automorph_src(w0 + i, g, log_n));
  } else {
    const ulonglong2* s2 = reinterpret_cast<const ulonglong2*>(src);
#pragma unroll
    for (int i = 0; i < W / 2; ++i) {
      const ulonglong2 v = at_u32(s2, (w0 >> 1) + i);
      x[2 * i] = v.x;
      x[2 * i + 1] = v.y;
    }
  }
  ip_inv_butterflies<G::RW, LOGB, AR, 0, W>(x, base, 0, col, twl, q);
  wave_lds_wait();  // the wave has read its columns' previous contents
#pragma unroll
  for (int i = 0; i < W; ++i) lds[ip_lds<LOGB>(base + i, col)] = x[i];
  wave_lds_wait();
  ip_inv_rounds_up<LOGB, AR, W, G::RW>(dst, lds, twl, tile, q, inv1);
}

}  // namespace nttc
}  // namespace ckks
