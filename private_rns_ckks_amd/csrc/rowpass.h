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

// Work item k (k < 8 >> R) of the calling thread in a register round of R
// stages at row bit pos.  Wave w takes the items of its own 2^(9-LOGB)
// columns (KC columns over THREADS / 64 waves), consecutive lanes taking
// consecutive items; for R = 3 this is the thread's column in every other
// round too, so each wave touches only its own columns of the LDS tile in
// every round of a pass, and the rounds need no workgroup barrier.
template <int R, int LOGB>
__device__ __forceinline__ void ip_item(int k, int pos, int& col, int& base) {
  constexpr int NB = 1 << (LOGB - R);  // items per column
  const int u = k * 64 + ((int)threadIdx.x & 63);
  col = ((int)threadIdx.x >> 6) * (1 << (9 - LOGB)) + u / NB;
  const int b = u % NB;
  base = ((b >> pos) << (pos + R)) | (b & ((1 << pos) - 1));
}

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
template <int R, int LOGB, int AR>
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
      for (int m = 0; m < half; ++m) ct_butterfly<AR>(x[i0 + m], x[i0 + m + half], w.x, w.y, q);
    }
  }
}

// One register round of R forward stages on row bits [POS, POS+R): item k of
// the thread (k < 8 >> R) is tid + k * THREADS; its words are rows
// base + (i << POS) of column col, read from global memory (src) or LDS and
// left in LDS or in x[].
template <int R, int POS, int LOGB, int AR, bool FROM_GLOBAL, bool TO_LDS>
__device__ __forceinline__ void ip_round(uint64_t (&x)[8], const uint64_t* src, uint64_t* lds, const ulonglong2* twl,
                                         uint32_t tile, int log_n, uint64_t q) {
  constexpr int T = IPRounds<LOGB>::THREADS;
  constexpr int NI = 8 >> R;
  uint64_t y[NI][1 << R];
  int col[NI], base[NI];
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    ip_item<R, LOGB>(k, POS, col[k], base[k]);
#pragma unroll
    for (int i = 0; i < (1 << R); ++i) {
      const int row = base[k] + (i << POS);
      y[k][i] = FROM_GLOBAL ? src[ip_word<LOGB>(tile, row, col[k])] : lds[ip_lds<LOGB>(row, col[k])];
    }
  }
#pragma unroll
  for (int k = 0; k < NI; ++k) {
    ip_butterflies<R, LOGB, AR>(y[k], base[k], POS, col[k], twl, q);
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
template <int LOGB, int AR>
__device__ __forceinline__ void ip_row_pass_first(const uint64_t* src, uint64_t* lds, const ulonglong2* twl,
                                                  uint32_t tile, int log_n, uint64_t q) {
  typedef IPRounds<LOGB> G;
  uint64_t unused[8];
  wave_lds_wait();  // the wave has read its columns' previous contents
  if constexpr (G::R1 > 0)
    ip_round<G::R1, LOGB - G::R1, LOGB, AR, true, true>(unused, src, lds, twl, tile, log_n, q);
  else
    ip_round<G::R2, G::R3, LOGB, AR, true, true>(unused, src, lds, twl, tile, log_n, q);
}
template <int LOGB, int AR>
__device__ __forceinline__ void ip_row_pass_rest(uint64_t (&x)[8], uint64_t* lds, const ulonglong2* twl,
                                                 uint32_t tile, int log_n, uint64_t q) {
  typedef IPRounds<LOGB> G;
  if constexpr (G::R1 > 0) {
    wave_lds_wait();
    ip_round<G::R2, G::R3, LOGB, AR, false, true>(x, nullptr, lds, twl, tile, log_n, q);
  }
  wave_lds_wait();
  ip_round<G::R3, 0, LOGB, AR, false, false>(x, nullptr, lds, twl, tile, log_n, q);
}

// R inverse (Gentleman-Sande) stages on the 2^R words of one item (rows
// base + (i << pos) of column col), highest stage first, twiddles from the
// LDS copy of the inverse table.  KDONE: stages of this pass already done
// (the bound of the lazy butterflies).
template <int R, int LOGB, int AR, int KDONE>
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
      const ulonglong2 w = twl[IPRounds<LOGB>::KC * ((1 << d) - 1) + (col << d) + (row >> (LOGB - d))];
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

// Inverse row pass of one limb on the tile: src holds canonical (or below
// 4q) words, dst receives the pass's output for the column pass that follows
// (below 4q: inv_row_out); with g nonzero the input is read through tau_g.
// Rounds on row bits 0-2 (8 consecutive words per thread, 16-byte loads, or
// word by word through tau_g), then 3.. and
// 6.. through the LDS tile; the last round's stores cover consecutive rows
// across the wave.
template <int LOGB, int AR>
__device__ __forceinline__ void ip_inv_row_pass(const uint64_t* src, uint64_t* dst, uint64_t* lds,
                                                const ulonglong2* twl, uint32_t tile, uint64_t q, uint64_t inv1,
                                                uint32_t g = 0, int log_n = 0) {
  typedef IPRounds<LOGB> G;
  constexpr int T = G::THREADS;
  int col, base;
  ip_item<3, LOGB>(0, 0, col, base);
  uint64_t x[8];
  const uint32_t w0 = ip_word<LOGB>(tile, base, col);
  if (g) {  // the input through tau_g (automorph.h): word j comes from word automorph_src(j, g)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = src[automorph_src(w0 + i, g, log_n)];
  } else {
    const ulonglong2* s2 = reinterpret_cast<const ulonglong2*>(src + w0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const ulonglong2 v = s2[i];
      x[2 * i] = v.x;
      x[2 * i + 1] = v.y;
    }
  }
  ip_inv_butterflies<3, LOGB, AR, 0>(x, base, 0, col, twl, q);
  wave_lds_wait();  // the wave has read its columns' previous contents
#pragma unroll
  for (int i = 0; i < 8; ++i) lds[ip_lds<LOGB>(base + i, col)] = x[i];
  wave_lds_wait();
  constexpr int N2 = 8 >> G::R2;
#pragma unroll
  for (int k = 0; k < N2; ++k) {
    int c, b;
    ip_item<G::R2, LOGB>(k, 3, c, b);
    uint64_t y[1 << G::R2];
#pragma unroll
    for (int i = 0; i < (1 << G::R2); ++i) y[i] = lds[ip_lds<LOGB>(b + (i << 3), c)];
    ip_inv_butterflies<G::R2, LOGB, AR, 3>(y, b, 3, c, twl, q);
#pragma unroll
    for (int i = 0; i < (1 << G::R2); ++i) {
      if constexpr (G::R1 == 0) dst[ip_word<LOGB>(tile, b + (i << 3), c)] = inv_row_out<AR>(y[i], q, inv1);
      else lds[ip_lds<LOGB>(b + (i << 3), c)] = y[i];
    }
  }
  if constexpr (G::R1 > 0) {
    wave_lds_wait();
    constexpr int N1 = 8 >> G::R1;
    constexpr int P1 = 3 + G::R2;
#pragma unroll
    for (int k = 0; k < N1; ++k) {
      int c, b;
      ip_item<G::R1, LOGB>(k, P1, c, b);
      uint64_t y[1 << G::R1];
#pragma unroll
      for (int i = 0; i < (1 << G::R1); ++i) y[i] = lds[ip_lds<LOGB>(b + (i << P1), c)];
      ip_inv_butterflies<G::R1, LOGB, AR, P1>(y, b, P1, c, twl, q);
#pragma unroll
      for (int i = 0; i < (1 << G::R1); ++i)
        dst[ip_word<LOGB>(tile, b + (i << P1), c)] = inv_row_out<AR>(y[i], q, inv1);
    }
  }
}

}  // namespace nttc
}  // namespace ckks
