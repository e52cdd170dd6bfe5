// Core of the negacyclic NTT passes on gfx950, shared by the plain transform
// and by the fused key-switch kernels.
//
// Transform (the reading used throughout): word j of the forward output is the
// input polynomial evaluated at psi^(2*brv(j)+1).  The forward transform is a
// chain of log N radix-2 Cooley-Tukey stages with the powers of psi merged
// into the twiddles (stage S, butterfly block b uses psi^brv(2^S + b)); the
// inverse is the Gentleman-Sande chain with psi^-brv(.) and a final 1/N.
//
// Decomposition.  A 2^16-word limb (512 KiB) does not fit the 160 KiB LDS of
// a CU, so the stages are split into two passes over memory:
//   column pass: the first LOGB stages of the forward transform only pair
//                words whose index agrees modulo N/2^LOGB, so each column of
//                2^LOGB words (stride N/2^LOGB) is independent;
//   row pass:    the remaining stages act inside contiguous blocks.
// The inverse runs the row pass first.  A workgroup owns a tile of 16 columns
// (column pass: 16 adjacent words per row, 128-byte segments) or 16 blocks
// (row pass) and runs its stages in two register rounds of radix 2^RA and
// 2^RB: each thread holds 2^R words and applies R stages in registers, with
// one LDS exchange between the rounds.  Loads and stores go straight between
// registers and memory where the lanes of a wave touch adjacent words;
// otherwise (first round of the inverse row pass, last round of the forward
// row pass) they are staged through LDS.
//
// Element I/O is a template policy (see PlainIO; j = word index within the
// limb), so a pass can gather its input (automorphism) or combine its output
// with other data (key-switch epilogue) without a separate trip through
// memory.
//
// Arithmetic ranges (template parameter AR, chosen per prime by fwd_ar /
// inv_ar):
//   AR_LAZY    forward q < 2^57: Shoup products with an approximate quotient
//              ([0, 4q)) and no reduction (values grow by at most 4q per
//              stage: 16 stages from [0, q) stay below 65q < 2^64); inverse
//              q < 2^54: the sum is not reduced (the bound doubles per stage
//              from 4q, 8 stages end below 2^10 q, each pass reduces once);
//   AR_HARVEY  q < 2^61: forward words in [0, 8q), inverse in [0, 4q), with
//              one conditional subtraction per butterfly;
//   AR_STRICT  q < 2^62: forward words in [0, 4q) and inverse in [0, 2q),
//              with exact-quotient Shoup products ([0, 2q)).
// The last pass reduces to [0, q).
#pragma once
#include "arith.h"
#include "internal.h"

namespace ckks {
namespace nttc {

constexpr int kCols = 16;
constexpr int kThreads = 256;

// global word index (within the limb) of tile element (row, col)
template <bool COLFAST>
__device__ __forceinline__ uint32_t tile_index(uint32_t tile, uint32_t row, uint32_t col, int logb, int log_n) {
  if (COLFAST) return tile * kCols + col + (row << (log_n - logb));
  return ((tile * kCols + col) << logb) + row;
}

// LDS position of tile element (row, col), unpadded (a 2^16 tile takes
// exactly 32 KiB, so five workgroups fit a CU's 160 KiB).  Column pass:
// row-major with row bit 0 flipped by row bit RB; row pass: column-major with
// the low 4 row bits XOR-ed with the next 4 and row bit 4 flipped by column
// bit 0.  In both register rounds and in the staging loops every 64-bit
// access of a wave then shares its bank pair with at most one other lane
// (the minimum for 64 lanes x 8 bytes on 64 four-byte banks).
template <bool COLFAST, int RB, int ROWS>
__device__ __forceinline__ int lds_index(int row, int col) {
  if (COLFAST) return (row ^ ((row >> RB) & 1)) * kCols + col;
  return col * ROWS + (row ^ ((row >> 4) & 15) ^ ((col & 1) << 4));
}
template <bool COLFAST, int RB, int ROWS>
constexpr int lds_words() {
  return ROWS * kCols;
}

__device__ __forceinline__ void load_tw(const uint64_t* tw, uint32_t ti, uint64_t& w, uint64_t& wp) {
  const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(tw + 2 * ti);
  w = v.x;
  wp = v.y;
}

// Element idx of an array whose base is the same across the wave, addressed
// as the base plus a 32-bit byte offset (idx * sizeof(T) below 2^32): the
// global load or store can then take the base from scalar registers and one
// offset register per lane, instead of a 64-bit address per lane.
template <class T>
__device__ __forceinline__ T& at_u32(T* base, uint32_t idx) {
  typedef typename std::conditional<std::is_const<T>::value, const char, char>::type Byte;
  uint32_t off = idx * (uint32_t)sizeof(T);
  asm volatile("" : "+v"(off));
  return *reinterpret_cast<T*>(reinterpret_cast<Byte*>(base) + off);
}

enum : int { AR_STRICT = 0, AR_HARVEY = 1, AR_LAZY = 2 };
__host__ __device__ inline int fwd_ar(uint64_t q) {
  return q < (1ull << 57) ? AR_LAZY : q < (1ull << 61) ? AR_HARVEY : AR_STRICT;
}
__host__ __device__ inline int inv_ar(uint64_t q) {
  return q < (1ull << 54) ? AR_LAZY : q < (1ull << 61) ? AR_HARVEY : AR_STRICT;
}

template <int AR>
__device__ __forceinline__ void ct_butterfly(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  if (AR == AR_STRICT) {  // words below 4q
    const uint64_t two_q = 2 * q;
    const uint64_t u = x >= two_q ? x - two_q : x;
    const uint64_t t = mul_shoup(y, w, wp, q);  // [0, 2q)
    x = u + t;
    y = u + two_q - t;
    return;
  }
  const uint64_t four_q = 4 * q;
  uint64_t u = x;
  if (AR == AR_HARVEY) u = u >= four_q ? u - four_q : u;
  const uint64_t t = mul_shoup_lazy(y, w, wp, q);  // [0, 4q)
  x = u + t;
  y = u + four_q - t;
}

__device__ __forceinline__ void gs_butterfly(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  const uint64_t four_q = 4 * q;
  const uint64_t s = x + y;
  const uint64_t d = x + four_q - y;
  x = s >= four_q ? s - four_q : s;
  y = mul_shoup_lazy_split(d, w, wp, q);
}

// Gentleman-Sande on words below 2q, for q < 2^62: sums below 4q.
__device__ __forceinline__ void gs_butterfly_strict(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q) {
  const uint64_t two_q = 2 * q;
  const uint64_t s = x + y;
  const uint64_t d = x + two_q - y;
  x = s >= two_q ? s - two_q : s;
  y = mul_shoup(d, w, wp, q);  // [0, 2q)
}

// Inverse butterfly of range AR; m: the lazy bound of the stage (AR_LAZY).
template <int AR>
__device__ __forceinline__ void gs_butterfly_ar(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q,
                                                uint64_t m);

// Gentleman-Sande without reducing the sum, for q < 2^54: with every word of
// the pass below m before the stage, the sum stays below 2m, x + m - y lies in
// (0, 2m) and the product below 4q, so m doubles per stage.  From words below
// 4q, 8 stages end below 2^10 q < 2^64; the pass reduces once at its end.
__device__ __forceinline__ void gs_butterfly_lazy(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q,
                                                  uint64_t m) {
  const uint64_t s = x + y;
  const uint64_t d = x + m - y;
  x = s;
  y = mul_shoup_lazy_split(d, w, wp, q);
}

template <int AR>
__device__ __forceinline__ void gs_butterfly_ar(uint64_t& x, uint64_t& y, uint64_t w, uint64_t wp, uint64_t q,
                                                uint64_t m) {
  if (AR == AR_LAZY) gs_butterfly_lazy(x, y, w, wp, q, m);
  else if (AR == AR_HARVEY) gs_butterfly(x, y, w, wp, q);
  else gs_butterfly_strict(x, y, w, wp, q);
}

// R stages in registers on the 2^R words x[] of one thread; the words are
// rows base + (i << pos) of column col.  Global stage of sub-stage s is
// s0 + logb - pos - R + s.
// With UTW the round's twiddles are the same for every thread of the
// workgroup (a column-pass round on row bits [pos, pos+R) whose base rows are
// below 2^pos, so the twiddle index depends on the group only): they are read
// with scalar loads into SGPRs.
typedef const __attribute__((address_space(4))) uint64_t* ConstTw;

// KDONE: stages of this pass already done (bound of the lazy inverse).
template <int R, bool INV, int AR, bool COLFAST, bool UTW = false, int KDONE = 0>
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
      uint64_t w, wp;
      if (UTW) {
        const uint32_t ti = (1u << S) + (((uint32_t)i0 << pos) >> (logb - S));
        const ConstTw twc = (ConstTw)tw;
        w = twc[2 * ti];
        wp = twc[2 * ti + 1];
      } else {
        const uint32_t j = tile_index<COLFAST>(tile, base + (i0 << pos), col, logb, log_n);
        load_tw(tw, (1u << S) + (j >> (log_n - S)), w, wp);
      }
#pragma unroll
      for (int m = 0; m < half; ++m) {
        if (INV) gs_butterfly_ar<AR>(x[i0 + m], x[i0 + m + half], w, wp, q, (4 * q) << (KDONE + ss));
        else ct_butterfly<AR>(x[i0 + m], x[i0 + m + half], w, wp, q);
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

// End-of-transform handling of the last pass.
struct Finish {
  int mode;        // 0: leave lazy (first pass), 1: reduce to [0,q), 2: inverse, times (w, wp) then reduce
  uint64_t w, wp;  // mode 2 multiplier
  uint64_t inv1;   // floor(2^64/q), forward reduction
};

// Pass geometry for N = 2^log_n: the column pass covers the first logb_col
// stages of the forward transform.
__host__ __device__ constexpr int logb_col(int log_n) { return (log_n + 1) / 2; }
__host__ __device__ constexpr int logb_row(int log_n) { return log_n - logb_col(log_n); }

// Tile word (column-major) handled by thread tid in step k of a staging loop:
// the workgroup sweeps the tile (WAVE = false), or each wave sweeps its own
// 64 * PER words (WAVE = true); either way consecutive lanes take
// consecutive words.
template <bool WAVE, int PER>
__device__ __forceinline__ int stage_index(int tid, int k) {
  return WAVE ? (tid >> 6) * (64 * PER) + k * 64 + (tid & 63) : tid + k * kThreads;
}

// The wave's LDS reads and writes so far are complete; the memory clobber
// keeps the compiler from moving LDS accesses across.  A wave runs in
// lockstep, so its lanes then see each other's writes without a barrier.
__device__ __forceinline__ void wave_lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// LOGN > 0 fixes log N at compile time (index arithmetic folds to constants);
// LOGN = 0 takes it from log_n_rt.
template <int RA, int RB, bool INV, bool COLFAST, int AR, int LOGN, class IO>
__device__ __forceinline__ void pass_body(const IO& io, uint64_t* lds, uint32_t tile, int log_n_rt,
                                          const uint64_t* tw, uint64_t q, const Finish& fin) {
  const int log_n = LOGN ? LOGN : log_n_rt;
  const uint32_t s0 = COLFAST ? 0u : (uint32_t)logb_col(log_n);  // row pass follows the column pass
  constexpr int LOGB = RA + RB;
  constexpr int ROWS = 1 << LOGB;
  constexpr int TILE = ROWS * kCols;
  const int tid = threadIdx.x;
  // first round: forward = high bits (pos RB, RA stages); inverse = low bits (pos 0, RB stages)
  constexpr int R1 = INV ? RB : RA;
  constexpr int R2 = INV ? RA : RB;
  const int pos1 = INV ? 0 : RB;
  const int pos2 = INV ? RB : 0;
  constexpr bool stage_in = INV && !COLFAST;   // inverse row pass: first round strided in memory
  constexpr bool stage_out = !INV && !COLFAST; // forward row pass: last round strided in memory
  constexpr int PER = TILE / kThreads;  // words per thread in the staging loops
  // When every thread takes part in the last round of the forward row pass,
  // wave w's threads hold exactly tile words [64 w PER, 64 (w+1) PER)
  // (column-major: e = col * ROWS + row), so each wave stores its own words
  // in coalesced order after waiting only for its own LDS writes, not for a
  // workgroup barrier (C2 forward row pass 123 against 127-129 us).
  constexpr bool wave_out = stage_out && kCols * (ROWS >> R2) == kThreads;
  if (stage_in) {
    // all loads first, then the LDS and side stores: keeps the loads in flight together
    uint64_t v[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + k * kThreads, row = e % ROWS, col = e / ROWS;
      v[k] = io.load(tile_index<COLFAST>(tile, row, col, LOGB, log_n));
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + k * kThreads, row = e % ROWS, col = e / ROWS;
      lds[lds_index<COLFAST, RB, ROWS>(row, col)] = v[k];
      io.after_load(tile_index<COLFAST>(tile, row, col, LOGB, log_n), v[k]);
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
                      : io.load(tile_index<COLFAST>(tile, row, col, LOGB, log_n));
    }
    round_regs<R1, INV, AR, COLFAST, COLFAST && !INV>(x, base, pos1, col, LOGB, tile, s0, log_n, tw, q);
    // each thread writes back exactly the words it read: no hazard with other threads
#pragma unroll
    for (int i = 0; i < (1 << R1); ++i) lds[lds_index<COLFAST, RB, ROWS>(base + (i << pos1), col)] = x[i];
  }
  // A row pass whose two rounds have the same radix and use every thread
  // keeps each thread on column tid / (ROWS >> R1) in both rounds, so the
  // exchange stays inside the wave's own columns.
  if constexpr (!COLFAST && R1 == R2 && kCols * (ROWS >> R1) == kThreads)
    wave_lds_wait();
  else
    __syncthreads();
  if (tid < kCols * (ROWS >> R2)) {
    int col, base;
    item_coords<COLFAST, R2, LOGB>(tid, pos2, col, base);
    uint64_t x[1 << R2];
#pragma unroll
    for (int i = 0; i < (1 << R2); ++i) x[i] = lds[lds_index<COLFAST, RB, ROWS>(base + (i << pos2), col)];
    round_regs<R2, INV, AR, COLFAST, COLFAST && INV, R1>(x, base, pos2, col, LOGB, tile, s0, log_n, tw, q);
    if (INV && AR == AR_LAZY && fin.mode != 2) {
      // lazy inverse: words below 2^10 q, reduced once.  After the first
      // pass [0, 2.5q) is enough (the next pass takes words below 4q).
      if (fin.mode == 0 && q > kReduceHiMin) {
#pragma unroll
        for (int i = 0; i < (1 << R2); ++i) x[i] = reduce_hi(x[i], q, (uint32_t)fin.inv1);
      } else {
#pragma unroll
        for (int i = 0; i < (1 << R2); ++i) x[i] = reduce64(x[i], q, fin.inv1);
      }
    } else if (fin.mode == 1) {
      if (INV) {
#pragma unroll
        for (int i = 0; i < (1 << R2); ++i) x[i] = reduce_4q(x[i], q);
      } else if (AR == AR_LAZY && q > kReduceHiMin && q < (1ull << 56)) {
        // lazy forward words lie below 65q < 2^63: reduce_hi leaves [0, 2q)
#pragma unroll
        for (int i = 0; i < (1 << R2); ++i) x[i] = reduce_2q(reduce_hi(x[i], q, (uint32_t)fin.inv1), q);
      } else {
#pragma unroll
        for (int i = 0; i < (1 << R2); ++i) x[i] = reduce64(x[i], q, fin.inv1);
      }
    } else if (fin.mode == 2) {
#pragma unroll
      for (int i = 0; i < (1 << R2); ++i) x[i] = reduce_4q(mul_shoup_lazy(x[i], fin.w, fin.wp, q), q);
    }
    if (stage_out) {
#pragma unroll
      for (int i = 0; i < (1 << R2); ++i) lds[lds_index<COLFAST, RB, ROWS>(base + (i << pos2), col)] = x[i];
    } else {
      typename IO::Ops ops[1 << R2];
#pragma unroll
      for (int i = 0; i < (1 << R2); ++i) ops[i] = io.fetch(tile_index<COLFAST>(tile, base + (i << pos2), col, LOGB, log_n));
#pragma unroll
      for (int i = 0; i < (1 << R2); ++i)
        io.store(tile_index<COLFAST>(tile, base + (i << pos2), col, LOGB, log_n), x[i], ops[i]);
    }
  }
  if (stage_out) {
    if constexpr (wave_out)
      wave_lds_wait();
    else
      __syncthreads();
    // fetch every operand of the epilogue before the first store
    typename IO::Ops ops[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = stage_index<wave_out, PER>(tid, k), row = e % ROWS, col = e / ROWS;
      ops[k] = io.fetch(tile_index<COLFAST>(tile, row, col, LOGB, log_n));
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = stage_index<wave_out, PER>(tid, k), row = e % ROWS, col = e / ROWS;
      io.store(tile_index<COLFAST>(tile, row, col, LOGB, log_n), lds[lds_index<COLFAST, RB, ROWS>(row, col)], ops[k]);
    }
  }
}

// Dispatch on the butterfly range of the prime.
template <int RA, int RB, bool INV, bool COLFAST, int LOGN, class IO>
__device__ __forceinline__ void run_pass(const IO& io, uint64_t* lds, uint32_t tile, int log_n,
                                         const uint64_t* tw, uint64_t q, const Finish& fin) {
  const int ar = INV ? inv_ar(q) : fwd_ar(q);
  if (ar == AR_LAZY)
    pass_body<RA, RB, INV, COLFAST, AR_LAZY, LOGN>(io, lds, tile, log_n, tw, q, fin);
  else if (ar == AR_HARVEY)
    pass_body<RA, RB, INV, COLFAST, AR_HARVEY, LOGN>(io, lds, tile, log_n, tw, q, fin);
  else
    pass_body<RA, RB, INV, COLFAST, AR_STRICT, LOGN>(io, lds, tile, log_n, tw, q, fin);
}

inline uint32_t pass_tiles(uint32_t n, int logb) { return n / ((1u << logb) * kCols); }

// Position of a row-pass workgroup in a (tiles, jobs, items) grid.  The chip
// hands workgroups to its 8 XCDs round-robin by linear id and each XCD has its
// own L2.  A row pass reads about twice its tile's data in twiddles, shared by
// every limb on the same prime, so the linear id is remapped to give each XCD
// a contiguous stretch of the order (tile fastest, then item, then job): the
// items that share a prime's twiddle table then run back to back on one L2,
// while the workgroups in flight still cover contiguous addresses.
constexpr uint32_t kXcds = 8;
struct GridPos {
  uint32_t tile;
  int job, item;
};
// Start of part c when n things are split into kXcds near-equal contiguous
// parts (the first n % kXcds parts one longer).
__device__ __forceinline__ uint32_t xcd_part_start(uint32_t c, uint32_t n) {
  const uint32_t m = n / kXcds, r = n % kXcds;
  return c < r ? c * (m + 1) : r * (m + 1) + (c - r) * m;
}
// ITEMS_FIRST puts the items of one (tile, job) next to each other instead:
// for the key inner product, whose items often share one key (a
// relinearisation key, or one rotation key for a whole batch), so that each
// key tile is fetched once for all of them.
template <bool ITEMS_FIRST = false>
__device__ __forceinline__ GridPos row_grid_pos() {
  const uint32_t gx = gridDim.x, gy = gridDim.y, gz = gridDim.z;
  const uint32_t b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const uint32_t logical = xcd_part_start(b % kXcds, gx * gy * gz) + b / kXcds;
  GridPos p;
  uint32_t jl;
  if (ITEMS_FIRST) {
    p.item = (int)(logical % gz);
    p.tile = (logical / gz) % gx;
    jl = logical / gz / gx;
  } else {
    p.tile = logical % gx;
    const uint32_t rest = logical / gx;
    p.item = (int)(rest % gz);
    jl = rest / gz;
  }
  // jobs in the order 0, 8, 16, ..., 1, 9, 17, ...: every XCD gets jobs from
  // across the range (the special primes, at the end, cost more per limb)
  const uint32_t m = gy / kXcds, r = gy % kXcds;
  uint32_t cls, idx;
  if (jl < r * (m + 1)) {
    cls = jl / (m + 1);
    idx = jl % (m + 1);
  } else {
    cls = r + (jl - r * (m + 1)) / m;
    idx = (jl - r * (m + 1)) % m;
  }
  p.job = (int)(cls + kXcds * idx);
  return p;
}

// Kernel instance for a pass of 2^logb rows at N = 2^log_n: N = 2^16 gets a
// compile-time specialisation, other sizes the generic one.
#define CKKS_PICK_PASS(kern, log_n, logb, ...)                   \
  ((log_n) == 16 && (logb) == 8 ? kern<4, 4, 16, ##__VA_ARGS__>  \
   : (logb) == 5              ? kern<3, 2, 0, ##__VA_ARGS__>   \
   : (logb) == 6              ? kern<3, 3, 0, ##__VA_ARGS__>   \
   : (logb) == 7              ? kern<4, 3, 0, ##__VA_ARGS__>   \
   : (logb) == 8              ? kern<4, 4, 0, ##__VA_ARGS__>   \
                              : nullptr)

// Element I/O policy.  load(j) supplies input word j; after_load(j, v) runs
// once per word after all loads of a staging loop (side outputs); fetch(j)
// reads whatever the store of word j needs and store(j, v, ops) writes the
// result -- every fetch of a loop is issued before its first store.
struct NoOps {};

struct PlainIO {
  typedef NoOps Ops;
  const uint64_t* src;
  uint64_t* dst;
  __device__ __forceinline__ uint64_t load(uint32_t j) const { return src[j]; }
  __device__ __forceinline__ void after_load(uint32_t, uint64_t) const {}
  __device__ __forceinline__ Ops fetch(uint32_t) const { return Ops(); }
  __device__ __forceinline__ void store(uint32_t j, uint64_t v, const Ops&) const { dst[j] = v; }
};

}  // namespace nttc
}  // namespace ckks
