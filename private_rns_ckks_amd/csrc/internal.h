// Internal declarations shared by the library's translation units: the
// context (device tables, workspace), error reporting and kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/ckks.h"

namespace ckks {

// Per-prime constants read by the kernels (one entry per basis prime).
struct PrimeConst {
  uint64_t q;
  uint64_t inv1;   // floor(2^64 / q)
  uint64_t r64;    // 2^64 mod q
  uint64_t r64p;   // Shoup quotient of r64
  uint64_t ninv;   // N^-1 mod q
  uint64_t ninvp;  // Shoup quotient of ninv
  uint64_t mprime; // -q^-1 mod 2^64 (Montgomery reduction)
  uint64_t pad;
};

// Basis-conversion constants for ModUp of digit j at level l (device copy at
// ctx->d_modup + offset).  Layout of the flat block (uint64 words):
//   [0, 2a)                : {[qhat_i^-1 * N^-1]_{q_i}, Shoup} for the a digit limbs
//   [2a, 2a + a*next)      : [qhat_i]_{m_t}, row i, column t over the extended
//                            basis at level l (next = l+1+K); unused in-digit columns are 0
// Basis-conversion source count rounded up to the kernels' unrolled count.
inline int conv_rows(uint32_t sources) { return sources <= 8 ? 8 : 16; }

struct ModUpEntry {
  int lo, hi;       // digit limbs [lo, hi)
  size_t offset;    // word offset into d_modup
};

// ModDown / rescale constants (flat device block d_moddown):
//   [0, 2K)            : {[phat_k^-1 * N^-1]_{p_k}, Shoup}
//   [2K, 2K + K*L)     : [phat_k * P^-1]_{q_i}, row k, column i
//   [.., + 2L)         : {[P^-1]_{q_i}, Shoup}
//   [.., + 2L)         : {[2^64 P^-1]_{q_i}, Shoup} (Montgomery sums times P^-1 in one product)
struct ModDownLayout {
  size_t phinv, conv, pinv, pinv64;
};

// Kernel timing trace (see ckks_trace_begin): HIP event pairs recorded on the
// launch stream around every launch of one kernel family.
struct TraceState {
  std::string name;                // family being traced, "" = off
  std::vector<hipEvent_t> pool;    // 2 events per traced launch
  size_t used = 0;
  double units = 0;                // algorithmic work units of the traced launches
};

struct Ctx {
  int device = 0;
  uint32_t log_n = 0, N = 0, L = 0, K = 0, dnum = 0, alpha = 0;
  std::vector<uint64_t> mod, psi;  // host copies, L+K entries
  // Some prime is at least 2^60: the dot-product kernels use full-width
  // 64x64-bit products instead of 30-bit halves.
  bool wide = false;
  PrimeConst* d_prime = nullptr;   // [L+K]
  uint64_t* d_tw_fwd = nullptr;    // [L+K][N][2] {psi^brv(k), Shoup}
  uint64_t* d_tw_inv = nullptr;    // [L+K][N][2] {psi^-brv(k), Shoup}
  uint64_t* d_modup = nullptr;
  std::vector<std::vector<ModUpEntry>> modup;  // [level][digit]
  uint64_t* d_moddown = nullptr;
  ModDownLayout md{};
  uint64_t* d_rescale = nullptr;  // [L][L][4]: for level l, limb i < l: {ql^-1, Shoup, ql mod q_i, 0}
  uint64_t* ws = nullptr;         // workspace
  size_t ws_words = 0;
  uint64_t* aux = nullptr;        // intermediate operands of composite calls (BSGS matvec)
  size_t aux_words = 0;
  TraceState trace;
  // Set while an allocation-free call runs: tracing records no events then
  // (creating them could allocate).
  bool no_alloc = false;
  // Sequence number of the key-switch chunk being dumped (CKKS_DEBUG_DUMP),
  // or -1 when dumping is off.
  int dump_seq = -1;
  // Internal streams (default priority) on which consecutive chunks of a
  // batch run concurrently, forked from and joined back to the caller's
  // stream with events; created on first use.
  static constexpr int kMaxLanes = 3;
  hipStream_t lane[kMaxLanes] = {};
  hipEvent_t fork_ev = nullptr, join_ev[kMaxLanes] = {};

  int beta(int level) const { return (level + 1 + (int)alpha - 1) / (int)alpha; }
  // basis index of extended limb t at level l (q_0..q_l, then p_0..p_{K-1})
  int ext_prime(int level, int t) const { return t <= level ? t : (int)L + (t - level - 1); }
};

// ---- errors -----------------------------------------------------------------
int set_error(int code, const std::string& msg);
#define CKKS_HIP_CHECK(expr)                                                            \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return set_error(CKKS_EHIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

int ensure_workspace(Ctx* c, size_t words);
int ensure_aux(Ctx* c, size_t words);
int ensure_lanes(Ctx* c);

// Records the start event (if `family` is being traced) on construction and
// the stop event on destruction; wrap exactly one kernel launch.
class TraceScope {
 public:
  TraceScope(Ctx* c, hipStream_t s, const char* family, double units);
  ~TraceScope();

 private:
  Ctx* c_;
  hipStream_t s_;
  bool on_;
};

// ---- NTT ----------------------------------------------------------------------
constexpr int kMaxJobs = 160;

// A list of limb transforms applied to `batch` polynomials: job i reads limb
// src_limb[i] of every batch item (src + b*src_bstride + src_limb[i]*N) and
// writes limb dst_limb[i] (dst + b*dst_bstride + dst_limb[i]*N), modulo basis
// prime prime[i].
struct NttJobs {
  int n = 0;
  uint16_t src_limb[kMaxJobs];
  uint16_t dst_limb[kMaxJobs];
  uint8_t prime[kMaxJobs];
  void add(int s, int d, int p) {
    src_limb[n] = (uint16_t)s;
    dst_limb[n] = (uint16_t)d;
    prime[n] = (uint8_t)p;
    ++n;
  }
};

// Forward (coefficient -> NTT form) or inverse transform of every job.
// inverse && !scale leaves out the 1/N factor (callers fold it into a later
// constant).  Outputs are fully reduced.  src may equal dst.
int ntt_run(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
            int batch, const NttJobs& jobs, bool inverse, bool scale);
// One pass only: forward first = column pass, forward second = row pass;
// inverse first = row pass, inverse second = column pass.  The second pass
// reduces to [0, q) (inverse: after the optional multiply, scale_mode as in
// ntt_run_scaled).  src may equal dst.
int ntt_pass_only(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
                  int batch, const NttJobs& jobs, bool inverse, bool first, int scale_mode, const uint64_t* scale_tab,
                  const uint32_t* scale_off);
// As ntt_run; an inverse transform ends with a multiply by 1/N (scale_mode 1)
// or by the per-job constant {w, w'} at scale_tab + scale_off[job] (mode 2).
int ntt_run_scaled(Ctx* c, hipStream_t s, const uint64_t* src, uint64_t* dst, size_t src_bstride, size_t dst_bstride,
                   int batch, const NttJobs& jobs, bool inverse, int scale_mode, const uint64_t* scale_tab,
                   const uint32_t* scale_off);

}  // namespace ckks

// The opaque handle of the C interface is the context itself.
struct ckks_ctx : public ckks::Ctx {};
