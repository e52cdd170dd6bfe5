// Context creation: parameter checks, prime search, and the per-prime device
// tables (twiddles, Shoup quotients, basis-conversion constants).
#include <string.h>

#include <new>

#include "host_math.h"
#include "internal.h"
#include "kernels.h"

namespace ckks {

static thread_local std::string g_last_error;

int set_error(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

// Grows a context-owned device buffer; the device is synchronised before the
// old buffer is freed, since queued work may still use it.
static int grow(uint64_t*& buf, size_t& have, size_t words, const char* what) {
  if (words <= have) return CKKS_OK;
  if (buf) {
    CKKS_HIP_CHECK(hipDeviceSynchronize());
    CKKS_HIP_CHECK(hipFree(buf));
    buf = nullptr;
    have = 0;
  }
  if (hipMalloc((void**)&buf, words * sizeof(uint64_t)) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(CKKS_ENOMEM, std::string(what) + " allocation of " + std::to_string(words * 8) + " bytes failed");
  }
  have = words;
  return CKKS_OK;
}

int ensure_workspace(Ctx* c, size_t words) { return grow(c->ws, c->ws_words, words, "workspace"); }
int ensure_aux(Ctx* c, size_t words) { return grow(c->aux, c->aux_words, words, "operand buffer"); }

TraceScope::TraceScope(Ctx* c, hipStream_t s, const char* family, double units)
    : c_(c), s_(s), on_(!c->no_alloc && !c->trace.name.empty() && c->trace.name == family) {
  if (!on_) return;
  TraceState& t = c->trace;
  while (t.pool.size() < t.used + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      on_ = false;
      return;
    }
    t.pool.push_back(e);
  }
  (void)hipEventRecord(t.pool[t.used], s);
  t.units += units;
}

TraceScope::~TraceScope() {
  if (!on_) return;
  (void)hipEventRecord(c_->trace.pool[c_->trace.used + 1], s_);
  c_->trace.used += 2;
}

static int validate(const ckks_params* p) {
  using namespace host;
  if (!p) return set_error(CKKS_EPARAM, "params is NULL");
  if (p->log_n < 10 || p->log_n > 16) return set_error(CKKS_EPARAM, "log_n must be in [10, 16]");
  if (p->n_q < 1 || p->n_q > 64) return set_error(CKKS_EPARAM, "n_q must be in [1, 64]");
  if (p->n_p > 16) return set_error(CKKS_EPARAM, "n_p must be at most 16");
  if (p->dnum < 1 || p->dnum > p->n_q) return set_error(CKKS_EPARAM, "dnum must be in [1, n_q]");
  uint32_t alpha = (p->n_q + p->dnum - 1) / p->dnum;
  if (p->n_p > 0 && alpha > 16) return set_error(CKKS_EPARAM, "digit size ceil(n_q/dnum) must be at most 16");
  if (p->n_p > 0 && p->n_p != alpha) return set_error(CKKS_EPARAM, "n_p must equal ceil(n_q/dnum)");
  if (!p->q || (p->n_p && !p->p)) return set_error(CKKS_EPARAM, "prime array is NULL");
  const uint64_t two_n = 2ull << p->log_n;
  std::vector<uint64_t> all(p->q, p->q + p->n_q);
  if (p->n_p) all.insert(all.end(), p->p, p->p + p->n_p);
  for (size_t i = 0; i < all.size(); ++i) {
    uint64_t m = all[i];
    if (m >= (1ull << 62)) return set_error(CKKS_EPARAM, "prime " + std::to_string(m) + " is not below 2^62");
    if (m % two_n != 1) return set_error(CKKS_EPARAM, "prime " + std::to_string(m) + " is not 1 mod 2N");
    if (!is_prime(m)) return set_error(CKKS_EPARAM, std::to_string(m) + " is not prime");
    for (size_t j = 0; j < i; ++j)
      if (all[j] == m) return set_error(CKKS_EPARAM, "primes must be distinct");
    if (p->psi) {
      uint64_t r = p->psi[i];
      if (r == 0 || r >= m || powmod(r, 1ull << p->log_n, m) != m - 1)
        return set_error(CKKS_EPARAM, "psi[" + std::to_string(i) + "] is not a primitive 2N-th root");
    }
  }
  return CKKS_OK;
}

static int upload(void** dst, const void* src, size_t bytes) {
  if (hipMalloc(dst, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return set_error(CKKS_ENOMEM, "table allocation failed");
  }
  CKKS_HIP_CHECK(hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice));
  return CKKS_OK;
}

int ensure_lanes(Ctx* c) {
  if (c->lane[0]) return CKKS_OK;
  for (int i = 0; i < Ctx::kMaxLanes; ++i) {
    CKKS_HIP_CHECK(hipStreamCreateWithFlags(&c->lane[i], hipStreamNonBlocking));
    CKKS_HIP_CHECK(hipEventCreateWithFlags(&c->join_ev[i], hipEventDisableTiming));
  }
  CKKS_HIP_CHECK(hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming));
  return CKKS_OK;
}

static void destroy(Ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  for (hipEvent_t e : c->trace.pool) (void)hipEventDestroy(e);
  for (int i = 0; i < Ctx::kMaxLanes; ++i) {
    if (c->lane[i]) (void)hipStreamDestroy(c->lane[i]);
    if (c->join_ev[i]) (void)hipEventDestroy(c->join_ev[i]);
  }
  if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
  void* bufs[] = {c->d_prime, c->d_tw_fwd, c->d_tw_inv, c->d_modup, c->d_moddown, c->d_rescale, c->ws, c->aux};
  for (void* b : bufs)
    if (b) (void)hipFree(b);
  delete c;
}

static int build_tables(Ctx* c) {
  using namespace host;
  const uint32_t N = c->N, LK = c->L + c->K;
  // per-prime constants
  std::vector<PrimeConst> pc(LK);
  for (uint32_t i = 0; i < LK; ++i) {
    uint64_t m = c->mod[i];
    PrimeConst& k = pc[i];
    memset(&k, 0, sizeof(k));
    k.q = m;
    k.inv1 = (uint64_t)((~(u128)0 >> 64) / m);  // floor((2^64 - 1) / m) = floor(2^64 / m) for non-powers of 2
    k.r64 = (uint64_t)(((u128)1 << 64) % m);
    k.r64p = shoup(k.r64, m);
    k.ninv = invmod(N % m, m);
    k.ninvp = shoup(k.ninv, m);
    uint64_t inv = m;  // Newton iteration: inverse of odd m modulo 2^64
    for (int it = 0; it < 6; ++it) inv *= 2 - m * inv;
    k.mprime = 0 - inv;
  }
  int rc = upload((void**)&c->d_prime, pc.data(), pc.size() * sizeof(PrimeConst));
  if (rc) return rc;
  // twiddles
  std::vector<uint64_t> fw((size_t)LK * N * 2), iv((size_t)LK * N * 2), pw(N), ipw(N);
  for (uint32_t i = 0; i < LK; ++i) {
    uint64_t m = c->mod[i], psi = c->psi[i], psi_inv = invmod(psi, m);
    pw[0] = ipw[0] = 1;
    for (uint32_t e = 1; e < N; ++e) {
      pw[e] = mulmod(pw[e - 1], psi, m);
      ipw[e] = mulmod(ipw[e - 1], psi_inv, m);
    }
    for (uint32_t k = 0; k < N; ++k) {
      uint32_t r = bit_reverse(k, (int)c->log_n);
      size_t o = ((size_t)i * N + k) * 2;
      fw[o] = pw[r];
      fw[o + 1] = shoup(pw[r], m);
      iv[o] = ipw[r];
      iv[o + 1] = shoup(ipw[r], m);
    }
  }
  if ((rc = upload((void**)&c->d_tw_fwd, fw.data(), fw.size() * 8))) return rc;
  if ((rc = upload((void**)&c->d_tw_inv, iv.data(), iv.size() * 8))) return rc;
  if (c->K == 0) return CKKS_OK;

  // Basis-conversion constants are stored split, lo30 | (v >> 30) << 32: the
  // operand form of the 30-bit split multiply-accumulate (constants below
  // 2^60); the full-width kernels reassemble the value (below 2^62).
  auto split30 = [](uint64_t v) { return (v & 0x3fffffffull) | ((v >> 30) << 32); };
  // ModUp constants per (level, digit)
  std::vector<uint64_t> mu;
  c->modup.assign(c->L, {});
  for (uint32_t level = 0; level < c->L; ++level) {
    const int next = (int)level + 1 + (int)c->K;
    for (int j = 0; j < c->beta((int)level); ++j) {
      ModUpEntry en;
      en.lo = j * (int)c->alpha;
      en.hi = std::min((j + 1) * (int)c->alpha, (int)level + 1);
      en.offset = mu.size();
      const int a = en.hi - en.lo;
      for (int x = 0; x < a; ++x) {
        uint64_t qi = c->mod[en.lo + x], prod = 1;
        for (int y = 0; y < a; ++y)
          if (y != x) prod = mulmod(prod, c->mod[en.lo + y] % qi, qi);
        uint64_t v = mulmod(invmod(prod, qi), invmod(N % qi, qi), qi);
        mu.push_back(v);
        mu.push_back(shoup(v, qi));
      }
      // rows for x >= a are zero: the kernel always runs conv_rows(alpha) sources
      for (int x = 0; x < conv_rows(c->alpha); ++x) {
        for (int t = 0; t < next; ++t) {
          if (x >= a || (t >= en.lo && t < en.hi)) {
            mu.push_back(0);
            continue;
          }
          uint64_t mt = c->mod[c->ext_prime((int)level, t)], prod = 1;
          for (int y = 0; y < a; ++y)
            if (y != x) prod = mulmod(prod, c->mod[en.lo + y] % mt, mt);
          mu.push_back(split30(prod));
        }
      }
      c->modup[level].push_back(en);
    }
  }
  if ((rc = upload((void**)&c->d_modup, mu.data(), mu.size() * 8))) return rc;

  // ModDown constants
  std::vector<uint64_t> md;
  const uint32_t K = c->K, L = c->L;
  c->md.phinv = md.size();
  for (uint32_t k = 0; k < K; ++k) {
    uint64_t pk = c->mod[L + k], prod = 1;
    for (uint32_t y = 0; y < K; ++y)
      if (y != k) prod = mulmod(prod, c->mod[L + y] % pk, pk);
    uint64_t v = mulmod(invmod(prod, pk), invmod(N % pk, pk), pk);
    md.push_back(v);
    md.push_back(shoup(v, pk));
  }
  c->md.conv = md.size();
  for (uint32_t k = 0; k < (uint32_t)conv_rows(K); ++k)  // rows k >= K are zero
    for (uint32_t i = 0; i < L; ++i)
      md.push_back(k < K ? split30(invmod(c->mod[L + k] % c->mod[i], c->mod[i])) : 0);  // phat_k / P = 1/p_k
  c->md.pinv = md.size();
  for (uint32_t i = 0; i < L; ++i) {
    uint64_t qi = c->mod[i], prod = 1;
    for (uint32_t k = 0; k < K; ++k) prod = mulmod(prod, c->mod[L + k] % qi, qi);
    uint64_t v = invmod(prod, qi);
    md.push_back(v);
    md.push_back(shoup(v, qi));
  }
  c->md.pinv64 = md.size();
  for (uint32_t i = 0; i < L; ++i) {
    const uint64_t qi = c->mod[i];
    const uint64_t v = mulmod((uint64_t)(((u128)1 << 64) % qi), md[c->md.pinv + 2 * i], qi);
    md.push_back(v);
    md.push_back(shoup(v, qi));
  }
  if ((rc = upload((void**)&c->d_moddown, md.data(), md.size() * 8))) return rc;
  return CKKS_OK;
}

static int build_rescale(Ctx* c) {
  using namespace host;
  const uint32_t L = c->L;
  std::vector<uint64_t> rs((size_t)L * L * 4, 0);
  for (uint32_t l = 1; l < L; ++l)
    for (uint32_t i = 0; i < l; ++i) {
      uint64_t qi = c->mod[i], ql = c->mod[l] % qi;
      uint64_t inv = invmod(ql, qi);
      size_t o = ((size_t)l * L + i) * 4;
      rs[o] = inv;
      rs[o + 1] = shoup(inv, qi);
      rs[o + 2] = ql;
    }
  return upload((void**)&c->d_rescale, rs.data(), rs.size() * 8);
}

}  // namespace ckks

using namespace ckks;

extern "C" {

const char* ckks_strerror(int status) {
  switch (status) {
    case CKKS_OK: return "ok";
    case CKKS_EINVAL: return "invalid argument";
    case CKKS_ERANGE: return "level or limb range out of range";
    case CKKS_ENOMEM: return "out of memory";
    case CKKS_EHIP: return "HIP runtime error";
    case CKKS_EPARAM: return "invalid parameter set";
    case CKKS_EINTERNAL: return "internal error";
  }
  return "unknown status";
}

const char* ckks_last_error(void) { return g_last_error.c_str(); }

int ckks_find_primes(uint32_t log_n, uint32_t bits, uint32_t count, uint64_t* out) {
  if (!out) return set_error(CKKS_EINVAL, "out is NULL");
  if (log_n < 1 || log_n > 30 || bits > 62 || bits < log_n + 2)
    return set_error(CKKS_EPARAM, "bits must be in [log_n+2, 62]");
  const uint64_t two_n = 2ull << log_n;
  uint64_t c = (1ull << bits) - two_n + 1;
  uint32_t found = 0;
  while (found < count && c > two_n) {
    if (host::is_prime(c)) out[found++] = c;
    c -= two_n;
  }
  if (found < count) return set_error(CKKS_EPARAM, "not enough primes below 2^bits");
  return CKKS_OK;
}

int ckks_params_validate(const ckks_params* params) { return validate(params); }

int ckks_ctx_create(const ckks_params* params, int hip_device, ckks_ctx** out) {
  if (!out) return set_error(CKKS_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = validate(params);
  if (rc) return rc;
  ckks_ctx* c = new (std::nothrow) ckks_ctx();
  if (!c) return set_error(CKKS_ENOMEM, "host allocation failed");
  c->device = hip_device;
  hipError_t e = hipSetDevice(hip_device);
  if (e != hipSuccess) {
    delete c;
    return set_error(CKKS_EHIP, std::string("hipSetDevice: ") + hipGetErrorString(e));
  }
  c->log_n = params->log_n;
  c->N = 1u << params->log_n;
  c->L = params->n_q;
  c->K = params->n_p;
  c->dnum = params->dnum;
  c->alpha = (c->L + c->dnum - 1) / c->dnum;
  c->mod.assign(params->q, params->q + c->L);
  if (c->K) c->mod.insert(c->mod.end(), params->p, params->p + c->K);
  for (uint64_t m : c->mod) c->wide = c->wide || m >= (1ull << 60);
  for (uint32_t i = 0; i < c->L + c->K; ++i)
    c->psi.push_back(params->psi ? params->psi[i] : host::smallest_primitive_root_2n(c->mod[i], (int)c->log_n));
  if ((rc = build_tables(c)) || (rc = build_rescale(c)) || (rc = noalloc_init_device(hip_device))) {
    destroy(c);
    return rc;
  }
  *out = c;
  return CKKS_OK;
}

int ckks_ctx_destroy(ckks_ctx* ctx) {
  if (!ctx) return set_error(CKKS_EINVAL, "ctx is NULL");
  destroy(ctx);
  return CKKS_OK;
}

int ckks_trace_begin(ckks_ctx* ctx, const char* kernel) {
  if (!ctx) return set_error(CKKS_EINVAL, "ctx is NULL");
  ctx->trace.name = kernel ? kernel : "";
  ctx->trace.used = 0;
  ctx->trace.units = 0;
  return CKKS_OK;
}

int ckks_trace_end(ckks_ctx* ctx, ckks_trace_stats* out) {
  if (!ctx || !out) return set_error(CKKS_EINVAL, "NULL argument");
  TraceState& t = ctx->trace;
  out->launches = (int32_t)(t.used / 2);
  out->total_ms = 0;
  out->work_units = t.units;
  for (size_t i = 0; i + 1 < t.used; i += 2) {
    float ms = 0;
    CKKS_HIP_CHECK(hipEventSynchronize(t.pool[i + 1]));
    CKKS_HIP_CHECK(hipEventElapsedTime(&ms, t.pool[i], t.pool[i + 1]));
    out->total_ms += ms;
  }
  t.name.clear();
  t.used = 0;
  t.units = 0;
  return CKKS_OK;
}

int ckks_ctx_psi(const ckks_ctx* ctx, uint64_t* out) {
  if (!ctx || !out) return set_error(CKKS_EINVAL, "NULL argument");
  for (size_t i = 0; i < ctx->psi.size(); ++i) out[i] = ctx->psi[i];
  return CKKS_OK;
}

}  // extern "C"
