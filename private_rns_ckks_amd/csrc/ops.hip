// Host orchestration of the hot path and the C ABI compute entry points.
// The key-switch pipeline itself is in keyswitch.hip.  Batch items are
// processed in chunks (CKKS_CHUNK, default 4) so that one launch covers
// several ciphertexts, and consecutive chunks alternate between internal
// streams (CKKS_LANES, default 2) so their kernels overlap.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "host_math.h"
#include "kernels.h"

namespace ckks {

namespace {

// Tuning knobs, read once: CKKS_LANES (concurrent chunks of a batch, 1 to
// Ctx::kMaxLanes) and CKKS_CHUNK (items per chunk).
int g_lanes_default() {
  static int v = [] {
    const char* e = getenv("CKKS_LANES");
    int x = e ? atoi(e) : 2;
    return std::max(1, std::min(x, Ctx::kMaxLanes));
  }();
  return v;
}

int g_chunk_default() {
  static int v = [] {
    const char* e = getenv("CKKS_CHUNK");
    int x = e ? atoi(e) : 4;
    return std::max(1, std::min(x, kMaxChunk));
  }();
  return v;
}

uint32_t inv_mod_2n(uint32_t g, uint32_t two_n) {
  uint32_t x = g;  // Newton iteration for the inverse of an odd number modulo a power of two
  for (int i = 0; i < 5; ++i) x *= 2 - g * x;
  return x & (two_n - 1);
}

int check_level(const Ctx* c, int level) {
  if (level < 0 || level >= (int)c->L) return set_error(CKKS_ERANGE, "level out of range");
  return CKKS_OK;
}

int check_galois(const Ctx* c, uint32_t g) {
  if (!(g & 1) || g >= 2 * c->N) return set_error(CKKS_EINVAL, "galois element must be odd and below 2N");
  return CKKS_OK;
}

// Rescale of `batch` items: in [2][level+1][N] at in + b*in_stride -> out
// [2][level][N], plus acc (same layout as out, may equal it) when given.
int rescale_batch(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t in_stride, uint64_t* out, uint64_t out_stride,
                  int batch, int level, uint64_t* ws, uint64_t ws_words, const uint64_t* add0 = nullptr,
                  const uint64_t* acc = nullptr) {
  const uint32_t N = c->N;
  const uint64_t per = (uint64_t)N * (2 + 2 * level);
  const int chunk = (int)std::max<uint64_t>(1, std::min<uint64_t>(kMaxChunk, ws_words / per));
  for (int b0 = 0; b0 < batch; b0 += chunk) {
    const int n = std::min(chunk, batch - b0);
    uint64_t* V = ws;
    uint64_t* W = ws + 2ull * N;
    NttJobs jobs;
    for (int comp = 0; comp < 2; ++comp) jobs.add(comp * (level + 1) + level, comp, level);
    int rc = ntt_run(c, s, in + b0 * in_stride, V, in_stride, per, n, jobs, true, true);
    if (rc) return rc;
    // conversion and final combination fused into the forward NTT of w
    if ((rc = rescale_fused(c, s, in + b0 * in_stride, in_stride, V, per, W, per, out + b0 * out_stride, out_stride, n,
                            level, add0, acc ? acc + b0 * out_stride : nullptr, out_stride)))
      return rc;
  }
  return CKKS_OK;
}

// Chunks of a batch on `lanes` internal streams: fork_lanes makes them wait
// for the work already on s; join_lanes makes s wait for them (also after a
// failure, so no lane work escapes the caller's stream order).
int fork_lanes(Ctx* c, hipStream_t s, int lanes) {
  if (lanes < 2) return CKKS_OK;
  int rc = ensure_lanes(c);
  if (rc) return rc;
  CKKS_HIP_CHECK(hipEventRecord(c->fork_ev, s));
  for (int l = 0; l < lanes; ++l) CKKS_HIP_CHECK(hipStreamWaitEvent(c->lane[l], c->fork_ev, 0));
  return CKKS_OK;
}

int join_lanes(Ctx* c, hipStream_t s, int lanes, int rc) {
  if (lanes < 2) return rc;
  for (int l = 0; l < lanes; ++l) {
    CKKS_HIP_CHECK(hipEventRecord(c->join_ev[l], c->lane[l]));
    CKKS_HIP_CHECK(hipStreamWaitEvent(s, c->join_ev[l], 0));
  }
  return rc;
}

hipStream_t lane_stream(Ctx* c, hipStream_t s, int lanes, int k) { return lanes > 1 ? c->lane[k % lanes] : s; }

// Multiply, relinearise and (when `rescale`) rescale a batch: a item b at
// a + b*2(l+1)N; b item b at b + b*b_bstride with component stride b_comp (so
// b may be a higher-level ciphertext read at its first l+1 limbs).  add0:
// optional per-limb constant added to component 0 of the rescaled output;
// acc: optional ciphertexts (the output's layout, may be the output itself)
// added to the rescaled output.
static int mul_relin_rescale(Ctx* ctx, hipStream_t stream, const uint64_t* d_a, const uint64_t* d_b,
                             uint64_t b_bstride,
                             uint64_t b_comp, const uint64_t* d_rlk, uint64_t* d_out, int batch, int level,
                             bool rescale, const uint64_t* add0, const uint64_t* acc = nullptr) {
  if (batch == 0) return CKKS_OK;
  const uint32_t N = ctx->N;
  const int nq = level + 1;
  const uint64_t ct = 2ull * nq * N;
  const int chunk = g_chunk_default();
  const int n_chunks = (batch + chunk - 1) / chunk;
  const int lanes = std::min(n_chunks, g_lanes_default());
  const uint64_t ks = ks_ws_words(ctx, level);
  // per chunk: tensor output [3][nq][N] per item, relinearised [2][nq][N] per item, then key-switch scratch
  const uint64_t tens = 3ull * nq * N, rel = ct;
  const uint64_t rs_per = (uint64_t)N * (2 + 2 * level);
  const uint64_t region = chunk * (tens + rel + std::max(ks, rs_per));  // one lane's workspace
  int rc;
  if ((rc = ensure_workspace(ctx, region * lanes)) || (rc = fork_lanes(ctx, stream, lanes))) return rc;
  for (int k = 0; k < n_chunks && rc == CKKS_OK; ++k) {
    const int b0 = k * chunk, n = std::min(chunk, batch - b0);
    const hipStream_t ls = lane_stream(ctx, stream, lanes, k);
    uint64_t* D = ctx->ws + region * (k % lanes);
    uint64_t* R = D + chunk * tens;
    uint64_t* S = R + chunk * rel;
    TensorArgs ta;
    ta.a = d_a + b0 * ct;
    ta.b = d_b + b0 * b_bstride;
    ta.out = D;
    ta.in_bstride = ct;
    ta.b_bstride = b_bstride;
    ta.b_comp = b_comp;
    ta.out_bstride = tens;
    ta.prime = ctx->d_prime;
    ta.n = N;
    ta.level = level;
    if ((rc = launch_tensor(ctx, ls, ta, n))) break;
    KSItem items[kMaxChunk];
    for (int i = 0; i < n; ++i) {
      KSItem& it = items[i];
      it.d = D + i * tens + 2ull * nq * N;
      it.g = 0;
      it.evk = d_rlk;
      it.add[0] = D + i * tens;
      it.add[1] = D + i * tens + (uint64_t)nq * N;
      it.add_g = 0;
      it.accum = nullptr;
      it.out = rescale ? R + i * rel : d_out + (b0 + i) * ct;
    }
    if ((rc = ks_chunk(ctx, ls, level, n, items, tens, tens, 0, rel, nq, S))) break;
    if (rescale)
      rc = rescale_batch(ctx, ls, R, rel, d_out + b0 * 2ull * level * N, 2ull * level * N, n, level, S,
                         chunk * std::max(ks, rs_per), add0, acc ? acc + b0 * 2ull * level * N : nullptr);
  }
  return join_lanes(ctx, stream, lanes, rc);
}

// Key switching of rotation pieces: each piece is up to g_chunk_default()
// items at in + i*stride / out + i*stride (i < n), all rotated by g with one
// key.  Piece k runs on internal stream k % lanes with its own workspace, so
// one piece's memory-bound kernels overlap another's arithmetic-bound ones.
struct RotPiece {
  const uint64_t* in;
  uint64_t* out;
  uint64_t stride;
  int n;
  const uint32_t* g;           // item m: g[m * step]
  const uint64_t* const* evk;  // item m: evk[m * step]
  int step;                    // 1: per-item elements and keys, 0: one for all
};

// With fixed_ws the pieces run one after another on s with that workspace
// (no internal streams, nothing allocated); otherwise on the lanes with the
// context's workspace, grown as needed.
static int rotate_pieces(Ctx* c, hipStream_t s, const std::vector<RotPiece>& pieces, int level, unsigned flags,
                         int chunk, uint64_t* fixed_ws = nullptr) {
  const int nq = level + 1;
  const uint64_t per = ks_ws_words(c, level);
  int rc = CKKS_OK;
  const int lanes = fixed_ws ? 1 : (int)std::min<size_t>(pieces.size(), g_lanes_default());
  if (pieces.empty()) return CKKS_OK;
  uint64_t* ws = fixed_ws;
  if (!fixed_ws) {
    if ((rc = ensure_workspace(c, per * chunk * lanes)) || (rc = fork_lanes(c, s, lanes))) return rc;
    ws = c->ws;
  }
  for (size_t k = 0; k < pieces.size() && rc == CKKS_OK; ++k) {
    const RotPiece& pc = pieces[k];
    KSItem items[kMaxChunk];
    for (int m = 0; m < pc.n; ++m) {
      KSItem& it = items[m];
      it.d = pc.in + m * pc.stride + (uint64_t)nq * c->N;  // c1
      it.g = pc.g[m * pc.step];
      it.evk = pc.evk[m * pc.step];
      it.add[0] = pc.in + m * pc.stride;  // c0, gathered through g
      it.add[1] = nullptr;
      it.add_g = it.g;
      it.accum = (flags & CKKS_ROT_ACCUMULATE) ? pc.in + m * pc.stride : nullptr;
      it.out = pc.out + m * pc.stride;
    }
    rc = ks_chunk(c, lane_stream(c, s, lanes, (int)k), level, pc.n, items, pc.stride, pc.stride, pc.stride,
                  pc.stride, nq, ws + per * chunk * (k % lanes));
  }
  return join_lanes(c, s, lanes, rc);
}

// Batched rotation with contiguous input/output (item b at base + b*stride).
// Items with g == 1 are copied (or doubled when accumulating); the others are
// key-switched in pieces of consecutive items (at most g_chunk_default()).
int rotate_batch(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t* out, uint64_t stride, int batch, int level,
                 const uint32_t* g, const uint64_t* const* evk, unsigned flags, uint64_t* fixed_ws = nullptr,
                 uint64_t fixed_words = 0) {
  const int nq = level + 1;
  const uint64_t ct_words = 2ull * nq * c->N;
  const int chunk = fixed_ws ? (int)std::min<uint64_t>(kMaxChunk, fixed_words / ks_ws_words(c, level))
                             : g_chunk_default();
  if (chunk < 1) return set_error(CKKS_EINTERNAL, "workspace smaller than one item");
  int rc;
  std::vector<int> idx;
  for (int b = 0; b < batch; ++b) {
    if (g[b] == 1) {
      if (flags & CKKS_ROT_ACCUMULATE) {
        if ((rc = launch_add(c, s, in + b * stride, in + b * stride, out + b * stride, 1, nq, 2, 0))) return rc;
      } else {
        CKKS_HIP_CHECK(hipMemcpyAsync(out + b * stride, in + b * stride, ct_words * 8, hipMemcpyDeviceToDevice, s));
      }
    } else {
      idx.push_back(b);
    }
  }
  // consecutive runs of non-identity items share a stride
  std::vector<RotPiece> pieces;
  for (size_t p = 0; p < idx.size();) {
    size_t q = p + 1;
    while (q < idx.size() && q - p < (size_t)chunk && idx[q] == idx[q - 1] + 1) ++q;
    const int b = idx[p];
    pieces.push_back(RotPiece{in + b * stride, out + b * stride, stride, (int)(q - p), g + b, evk + b, 1});
    p = q;
  }
  return rotate_pieces(c, s, pieces, level, flags, chunk, fixed_ws);
}

// Giant steps of a BSGS product: rot[o][g] = Rot_g(inner[o][g]) for g >= 1
// (items at base + (o*n2 + g)*ct), in pieces of outputs that share one giant
// step, so the items of a piece share their key.
static int rotate_giant_steps(Ctx* c, hipStream_t s, const uint64_t* inner, uint64_t* rot, uint64_t ct, int n_out,
                              int n2, int level, const uint32_t* giant_galois, const uint64_t* const* d_evk_giant) {
  const int chunk = g_chunk_default();
  std::vector<RotPiece> pieces;
  for (int g = 1; g < n2; ++g)
    for (int o0 = 0; o0 < n_out; o0 += chunk) {
      RotPiece pc;
      pc.in = inner + ((uint64_t)o0 * n2 + g) * ct;
      pc.out = rot + ((uint64_t)o0 * n2 + g) * ct;
      pc.stride = (uint64_t)n2 * ct;
      pc.n = std::min(chunk, n_out - o0);
      pc.g = giant_galois + (g - 1);
      pc.evk = d_evk_giant + (g - 1);
      pc.step = 0;
      pieces.push_back(pc);
    }
  return rotate_pieces(c, s, pieces, level, 0, chunk);
}

// Hoisted rotations: input c (at in + c*in_stride, [2][l+1][N]) rotated by
// g[r] (key evk[r]) into out + c*out_in_stride + r*out_rot_stride.  Inputs are
// decomposed in groups of up to kMaxChunk on s; the rotations of each input
// then run in chunks alternating over the lanes.
int rotate_hoisted(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t in_stride, int n_in, int level, int n_rot,
                   const uint32_t* g, const uint64_t* const* evk, uint64_t* out, uint64_t out_in_stride,
                   uint64_t out_rot_stride) {
  const int nq = level + 1;
  const uint64_t ct_words = 2ull * nq * c->N;
  const uint64_t dec_per = ks_dec_words(c, level), back_per = ks_back_words(c, level);
  const int chunk = g_chunk_default();
  int rc;
  std::vector<int> rots;  // rotations that need a key switch
  for (int r = 0; r < n_rot; ++r) {
    if (g[r] != 1) {
      rots.push_back(r);
      continue;
    }
    for (int ci = 0; ci < n_in; ++ci)
      CKKS_HIP_CHECK(hipMemcpyAsync(out + ci * out_in_stride + r * out_rot_stride, in + ci * in_stride, ct_words * 8,
                                    hipMemcpyDeviceToDevice, s));
  }
  if (rots.empty() || n_in == 0) return CKKS_OK;
  const int group = std::min(n_in, kMaxChunk);
  const int per_input = ((int)rots.size() + chunk - 1) / chunk;
  const int lanes = std::min(per_input * n_in, g_lanes_default());
  if ((rc = ensure_workspace(c, dec_per * group + back_per * chunk * lanes))) return rc;
  uint64_t* dec = c->ws;
  uint64_t* back = c->ws + dec_per * group;
  int k = 0;  // chunk counter, for the lane choice
  for (int c0 = 0; c0 < n_in; c0 += group) {
    const int n = std::min(group, n_in - c0);
    if ((rc = ks_decompose(c, s, level, n, in + c0 * in_stride + (uint64_t)nq * c->N, in_stride, dec, dec_per)))
      return rc;
    if ((rc = fork_lanes(c, s, lanes))) return rc;
    for (int ci = c0; ci < c0 + n && rc == CKKS_OK; ++ci) {
      for (size_t p = 0; p < rots.size() && rc == CKKS_OK; p += chunk, ++k) {
        const int m = (int)std::min<size_t>(chunk, rots.size() - p);
        KSItem items[kMaxChunk];
        memset(items, 0, sizeof(items));
        for (int i = 0; i < m; ++i) {
          const int r = rots[p + i];
          items[i].g = g[r];
          items[i].evk = evk[r];
          items[i].add[0] = in + ci * in_stride;  // c0, gathered through g
          items[i].add_g = g[r];
          items[i].out = out + ci * out_in_stride + r * out_rot_stride;
        }
        // consecutive entries of rots are not always consecutive rotations:
        // output items must advance by one stride, so split at gaps
        int i0 = 0;
        while (i0 < m && rc == CKKS_OK) {
          int i1 = i0 + 1;
          while (i1 < m && rots[p + i1] == rots[p + i1 - 1] + 1) ++i1;
          rc = ks_hoisted_chunk(c, lane_stream(c, s, lanes, k), level, i1 - i0, items + i0,
                                dec + (uint64_t)(ci - c0) * dec_per, in + ci * in_stride + (uint64_t)nq * c->N,
                                out_rot_stride, back + back_per * chunk * (k % lanes));
          i0 = i1;
        }
      }
    }
    // the next group's decomposition overwrites dec: wait for this group's chunks
    rc = join_lanes(c, s, lanes, rc);
    if (rc) return rc;
  }
  return CKKS_OK;
}

}  // namespace
}  // namespace ckks

using namespace ckks;

// device buffers are read and written with 16-byte vector accesses
static bool misaligned(const void* p) { return ((uintptr_t)p & 15) != 0; }

// True when the word ranges [a, a + a_words) and [b, b + b_words) share a
// byte.  Outputs are written by some workgroups while other workgroups still
// read (and gather) the inputs, so an output that overlaps an input or a key
// would race; such calls are rejected before any launch.
static bool overlap(const void* a, uint64_t a_words, const void* b, uint64_t b_words) {
  if (!a || !b || !a_words || !b_words) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + b_words * 8 && b0 < a0 + a_words * 8;
}
#define REJECT_OVERLAP(a, an, b, bn, what) \
  if (overlap((a), (an), (b), (bn))) return set_error(CKKS_EINVAL, "output overlaps " what)

#define CTX_OR_FAIL(ctx)                                             \
  if (!(ctx)) return set_error(CKKS_EINVAL, "ctx is NULL");         \
  if (hipSetDevice((ctx)->device) != hipSuccess) return set_error(CKKS_EHIP, "hipSetDevice failed")

extern "C" {

int ckks_ntt(ckks_ctx* ctx, uint64_t* d_data, int npoly, int limb_begin, int n_limb, int inverse,
             ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_data || npoly < 0 || n_limb < 0) return set_error(CKKS_EINVAL, "bad data pointer or count");
  if (misaligned(d_data)) return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  if (limb_begin < 0 || limb_begin + n_limb > (int)(ctx->L + ctx->K)) return set_error(CKKS_ERANGE, "limb range outside the basis");
  if (npoly == 0 || n_limb == 0) return CKKS_OK;
  if (npoly > 65535) return set_error(CKKS_EINVAL, "npoly too large");
  NttJobs jobs;
  for (int i0 = 0; i0 < n_limb; i0 += kMaxJobs) {
    jobs.n = 0;
    const int nl = std::min(kMaxJobs, n_limb - i0);
    for (int i = 0; i < nl; ++i) jobs.add(i0 + i, i0 + i, limb_begin + i0 + i);
    int rc = ntt_run(ctx, stream, d_data, d_data, (uint64_t)n_limb * ctx->N, (uint64_t)n_limb * ctx->N, npoly, jobs,
                     inverse != 0, true);
    if (rc) return rc;
  }
  return CKKS_OK;
}

int ckks_automorph(ckks_ctx* ctx, const uint64_t* d_in, uint64_t* d_out, int npoly, int level, uint32_t galois_elt,
                   int domain, ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_in || !d_out || npoly < 0) return set_error(CKKS_EINVAL, "bad pointer or count");
  if (misaligned(d_in) || misaligned(d_out)) return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc || (rc = check_galois(ctx, galois_elt))) return rc;
  if (domain != 0 && domain != 1) return set_error(CKKS_EINVAL, "domain must be 0 (NTT) or 1 (coefficient)");
  if (npoly == 0) return CKKS_OK;
  const uint64_t pstride = (uint64_t)(level + 1) * ctx->N;
  REJECT_OVERLAP(d_out, pstride * npoly, d_in, pstride * npoly, "the input");
  if (domain == 0) return launch_automorph_ntt(ctx, stream, d_in, d_out, npoly, level + 1, pstride, galois_elt);
  return launch_automorph_coeff(ctx, stream, d_in, d_out, npoly, level + 1, pstride,
                                inv_mod_2n(galois_elt, 2 * ctx->N));
}

int ckks_keyswitch(ckks_ctx* ctx, const uint64_t* d_poly, const uint64_t* d_evk, uint64_t* d_out, int level,
                   ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_poly || !d_evk || !d_out) return set_error(CKKS_EINVAL, "NULL pointer");
  if (misaligned(d_poly) || misaligned(d_evk) || misaligned(d_out))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (ctx->K == 0) return set_error(CKKS_EPARAM, "key switching needs special primes");
  const uint64_t key_words = (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * ctx->N;
  REJECT_OVERLAP(d_out, 2ull * (level + 1) * ctx->N, d_poly, (uint64_t)(level + 1) * ctx->N, "the input");
  REJECT_OVERLAP(d_out, 2ull * (level + 1) * ctx->N, d_evk, key_words, "the key");
  if ((rc = ensure_workspace(ctx, ks_ws_words(ctx, level)))) return rc;
  KSItem it;
  memset(&it, 0, sizeof(it));
  it.d = d_poly;
  it.evk = d_evk;
  it.out = d_out;
  return ks_chunk(ctx, stream, level, 1, &it, 0, 0, 0, 0, level + 1, ctx->ws);
}

}  // extern "C"

namespace ckks {

int rotate_check(Ctx* ctx, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                 const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags) {
  if (!d_ct_in || !d_ct_out || batch < 0 || (batch > 0 && (!galois_elts || !d_evks)))
    return set_error(CKKS_EINVAL, "NULL pointer or bad batch");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (flags & ~CKKS_ROT_ACCUMULATE) return set_error(CKKS_EINVAL, "unknown flag");
  for (int b = 0; b < batch; ++b) {
    if ((rc = check_galois(ctx, galois_elts[b]))) return rc;
    if (galois_elts[b] != 1 && !d_evks[b]) return set_error(CKKS_EINVAL, "NULL key pointer");
    if (galois_elts[b] != 1 && misaligned(d_evks[b])) return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  }
  if (misaligned(d_ct_in) || misaligned(d_ct_out))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  if (batch > 0 && ctx->K == 0) return set_error(CKKS_EPARAM, "rotation needs special primes");
  const uint64_t ct_words = 2ull * (level + 1) * ctx->N * batch;
  const uint64_t key_words = (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * ctx->N;
  REJECT_OVERLAP(d_ct_out, ct_words, d_ct_in, ct_words, "the input");
  for (int b = 0; b < batch; ++b)
    if (galois_elts[b] != 1) REJECT_OVERLAP(d_ct_out, ct_words, d_evks[b], key_words, "a key");
  return CKKS_OK;
}

int rotate_fixed_ws(Ctx* ctx, hipStream_t s, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                    const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags, uint64_t* ws,
                    uint64_t ws_words) {
  return rotate_batch(ctx, s, d_ct_in, d_ct_out, 2ull * (level + 1) * ctx->N, batch, level, galois_elts, d_evks,
                      flags, ws, ws_words);
}

}  // namespace ckks

extern "C" {

int ckks_rotate(ckks_ctx* ctx, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags, ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  int rc = rotate_check(ctx, d_ct_in, d_ct_out, batch, level, galois_elts, d_evks, flags);
  if (rc) return rc;
  return rotate_batch(ctx, stream, d_ct_in, d_ct_out, 2ull * (level + 1) * ctx->N, batch, level, galois_elts, d_evks,
                      flags);
}

int ckks_rotate_hoisted(ckks_ctx* ctx, const uint64_t* d_ct_in, int n_in, int level, int n_rot,
                        const uint32_t* galois_elts, const uint64_t* const* d_evks, uint64_t* d_ct_out,
                        ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_ct_in || !d_ct_out || n_in < 0 || n_rot < 0 || (n_rot > 0 && (!galois_elts || !d_evks)))
    return set_error(CKKS_EINVAL, "NULL pointer or bad count");
  if (misaligned(d_ct_in) || misaligned(d_ct_out))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  for (int r = 0; r < n_rot; ++r) {
    if ((rc = check_galois(ctx, galois_elts[r]))) return rc;
    if (galois_elts[r] != 1 && (!d_evks[r] || misaligned(d_evks[r])))
      return set_error(CKKS_EINVAL, "NULL or misaligned key pointer");
  }
  if (n_rot > 0 && ctx->K == 0) return set_error(CKKS_EPARAM, "rotation needs special primes");
  const uint64_t ct = 2ull * (level + 1) * ctx->N;
  const uint64_t key_words = (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * ctx->N;
  REJECT_OVERLAP(d_ct_out, ct * n_in * n_rot, d_ct_in, ct * n_in, "the input");
  for (int r = 0; r < n_rot; ++r)
    if (galois_elts[r] != 1) REJECT_OVERLAP(d_ct_out, ct * n_in * n_rot, d_evks[r], key_words, "a key");
  return rotate_hoisted(ctx, stream, d_ct_in, ct, n_in, level, n_rot, galois_elts, d_evks, d_ct_out, n_rot * ct, ct);
}

int ckks_rescale(ckks_ctx* ctx, const uint64_t* d_in, uint64_t* d_out, int batch, int level, ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_in || !d_out || batch < 0) return set_error(CKKS_EINVAL, "NULL pointer or bad batch");
  if (misaligned(d_in) || misaligned(d_out)) return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (level == 0) return set_error(CKKS_ERANGE, "cannot rescale at level 0");
  REJECT_OVERLAP(d_out, 2ull * level * ctx->N * batch, d_in, 2ull * (level + 1) * ctx->N * batch, "the input");
  const uint64_t per = (uint64_t)ctx->N * (2 + 2 * level);
  if ((rc = ensure_workspace(ctx, per * std::min(batch, kMaxChunk)))) return rc;
  return rescale_batch(ctx, stream, d_in, 2ull * (level + 1) * ctx->N, d_out, 2ull * level * ctx->N, batch, level,
                       ctx->ws, ctx->ws_words);
}

int ckks_mul_relin_rescale(ckks_ctx* ctx, const uint64_t* d_a, const uint64_t* d_b, const uint64_t* d_rlk,
                           uint64_t* d_out, int batch, int level, unsigned flags, ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_a || !d_b || !d_rlk || !d_out || batch < 0) return set_error(CKKS_EINVAL, "NULL pointer or bad batch");
  if (misaligned(d_a) || misaligned(d_b) || misaligned(d_rlk) || misaligned(d_out))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (flags & ~CKKS_NO_RESCALE) return set_error(CKKS_EINVAL, "unknown flag");
  const bool rescale = !(flags & CKKS_NO_RESCALE);
  if (rescale && level == 0) return set_error(CKKS_ERANGE, "cannot rescale at level 0");
  if (ctx->K == 0) return set_error(CKKS_EPARAM, "relinearisation needs special primes");
  const uint64_t ct = 2ull * (level + 1) * ctx->N;
  const uint64_t out_words = 2ull * (rescale ? level : level + 1) * ctx->N * batch;
  const uint64_t key_words = (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * ctx->N;
  REJECT_OVERLAP(d_out, out_words, d_a, ct * batch, "an input");
  REJECT_OVERLAP(d_out, out_words, d_b, ct * batch, "an input");
  REJECT_OVERLAP(d_out, out_words, d_rlk, key_words, "the key");
  return mul_relin_rescale(ctx, stream, d_a, d_b, ct, (uint64_t)(level + 1) * ctx->N, d_rlk, d_out, batch, level,
                           rescale, nullptr);
}

// round(x) for |x| < 2^62, the same rounding (llround) as the reference
// evaluation; false when out of range.
static bool round_checked(double x, int64_t* out) {
  if (!(fabs(x) < 4611686018427387904.0)) return false;
  *out = llround(x);
  return true;
}

static uint64_t signed_mod(int64_t v, uint64_t m) {
  if (v >= 0) return (uint64_t)v % m;
  const uint64_t r = (uint64_t)(-(v + 1)) % m;  // -(v+1) >= 0 without overflow
  return r == m - 1 ? 0 : m - 1 - r;
}

int ckks_poly_eval(ckks_ctx* ctx, const uint64_t* d_ct_in, int batch, int level, double scale, const double* coeffs,
                   int degree, const uint64_t* d_rlk, uint64_t* d_ct_out, double* out_scale, ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_ct_in || !d_ct_out || !d_rlk || !coeffs || !out_scale || batch < 0)
    return set_error(CKKS_EINVAL, "NULL pointer or bad batch");
  if (misaligned(d_ct_in) || misaligned(d_ct_out) || misaligned(d_rlk))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (degree < 1 || degree > level) return set_error(CKKS_ERANGE, "degree must be 1..level");
  if (ctx->K == 0) return set_error(CKKS_EPARAM, "relinearisation needs special primes");
  const int d = degree;
  // constants and scales, in the order and arithmetic of the reference
  int64_t kmul, kadd[64];
  double s_acc = scale;
  bool ok = round_checked(coeffs[d] * (double)ctx->mod[level], &kmul);
  ok = ok && round_checked(coeffs[d - 1] * s_acc, &kadd[d - 1]);
  for (int k = d - 2, l = level - 1; k >= 0; --k, --l) {
    s_acc = s_acc * scale / (double)ctx->mod[l];
    ok = ok && round_checked(coeffs[k] * s_acc, &kadd[k]);
  }
  if (!ok) return set_error(CKKS_EINVAL, "a rounded polynomial constant reaches 2^62");
  *out_scale = s_acc;
  if (batch == 0) return CKKS_OK;
  const uint32_t N = ctx->N;
  const uint64_t in_ct = 2ull * (level + 1) * N, ct_l = 2ull * level * N;
  const uint64_t out_words = 2ull * (level - degree + 1) * N * batch;
  REJECT_OVERLAP(d_ct_out, out_words, d_ct_in, in_ct * batch, "the input");
  REJECT_OVERLAP(d_ct_out, out_words, d_rlk, (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * N, "the key");
  // operand buffers: the constant product at level `level` and two accumulators
  if ((rc = ensure_aux(ctx, batch * (in_ct + 2 * ct_l)))) return rc;
  uint64_t* T = ctx->aux;
  uint64_t* acc[2] = {T + batch * in_ct, T + batch * in_ct + batch * ct_l};
  // acc = c_d * x: times round(c_d * q_l) on every limb, then rescale
  {
    ConstMulArgs cm;
    cm.in = d_ct_in;
    cm.out = T;
    cm.in_bstride = in_ct;
    cm.out_bstride = in_ct;
    cm.prime = ctx->d_prime;
    cm.nl = level + 1;
    cm.log_n = (int)ctx->log_n;
    for (int i = 0; i <= level; ++i) {
      cm.k[i][0] = signed_mod(kmul, ctx->mod[i]);
      cm.k[i][1] = host::shoup(cm.k[i][0], ctx->mod[i]);
    }
    if ((rc = launch_const_mul(ctx, stream, cm, batch))) return rc;
  }
  uint64_t* dst = d == 1 ? d_ct_out : acc[0];
  const uint64_t rs_per = (uint64_t)N * (2 + 2 * level);
  if ((rc = ensure_workspace(ctx, rs_per * std::min(batch, kMaxChunk)))) return rc;
  // the constants enter in NTT form (the same value in every word of a limb),
  // added to component 0 by the final store of each rescale
  uint64_t cv[64];
  auto consts = [&](int lvl, int64_t v) {
    for (int i = 0; i <= lvl; ++i) cv[i] = signed_mod(v, ctx->mod[i]);
    return cv;
  };
  if ((rc = rescale_batch(ctx, stream, T, in_ct, dst, ct_l, batch, level, ctx->ws, ctx->ws_words,
                          consts(level - 1, kadd[d - 1]))))
    return rc;
  int l = level - 1;
  // Horner steps: acc = rescale(relin(acc * x)) + c_k, with x read at its
  // first l+1 limbs in place
  for (int k = d - 2, cur = 0; k >= 0; --k, cur ^= 1) {
    uint64_t* next = k == 0 ? d_ct_out : acc[cur ^ 1];
    if ((rc = mul_relin_rescale(ctx, stream, acc[cur], d_ct_in, in_ct, (uint64_t)(level + 1) * N, d_rlk, next,
                                batch, l, true, consts(l - 1, kadd[k]))))
      return rc;
    --l;
  }
  return CKKS_OK;
}

static int ceil_log2(int k) {
  int r = 0;
  while ((1 << r) < k) ++r;
  return r;
}

namespace {

int trim_coeffs(const double* c, int n) {
  while (n > 0 && c[n - 1] == 0.0) --n;
  return n;
}

// Depth-efficient evaluation of a power-basis polynomial on a chunk of items
// (see ckks_poly_eval_tree in include/ckks.h for the scheme).  Node results
// and the high parts' intermediates live on a stack carved from `arena`.
struct TreeEval {
  Ctx* ctx;
  hipStream_t s;
  const uint64_t* rlk;
  int level, n;                // input level, items in the chunk
  const uint64_t* y[8];        // y_j = x^(2^j): item b at y[j] + b*y_stride[j], level - j
  uint64_t y_stride[8];
  double sc[8];
  uint64_t* G;                 // constant-product scratch, [n][2][level+1][N]
  uint64_t* stack;
  uint64_t top, cap;           // words used / available on the stack
  bool bad;

  uint64_t ct_words(int t) const { return 2ull * (t + 1) * ctx->N; }
  int64_t rnd(double v) {
    int64_t r = 0;
    if (!round_checked(v, &r)) bad = true;
    return r;
  }
  void consts(int t, int64_t k, uint64_t* cv) const {
    for (int i = 0; i <= t; ++i) cv[i] = signed_mod(k, ctx->mod[i]);
  }

  // Same recursion as eval(), constants only.
  void check(const double* c, int nc, int t, double T) {
    if (nc == 0) return;
    if (nc <= 2) {
      if (nc == 2) rnd(c[1] * T * (double)ctx->mod[t + 1] / sc[0]);
      rnd(c[0] * T);
      return;
    }
    const int j = ceil_log2(nc), g = 1 << (j - 1);
    const int n_lo = trim_coeffs(c, g), n_hi = nc - g;
    if (n_lo >= 2) check(c, n_lo, t, T);
    else if (n_lo == 1) rnd(c[0] * T);
    if (n_hi == 1) rnd(c[g] * T * (double)ctx->mod[t + 1] / sc[j - 1]);
    else check(c + g, n_hi, t + 1, T * (double)ctx->mod[t + 1] / sc[j - 1]);
  }

  // out (= [n][2][t+1][N]) = K * y (limbs 0..t+1 of y, at level ly) rescaled
  // by q_(t+1), plus acc, plus the constant k0 on component 0.
  int scaled(const uint64_t* y, uint64_t ystride, int ly, int64_t K, int t, uint64_t* out, const uint64_t* acc,
             bool has_k0, int64_t k0) {
    const uint32_t N = ctx->N;
    TermMacArgs ta;
    memset(&ta, 0, sizeof(ta));
    ta.x[0] = y;
    ta.k[0] = K;
    ta.nt = 1;
    ta.out = G;
    ta.x_bstride = ystride;
    ta.x_comp = (uint64_t)(ly + 1) * N;
    ta.out_bstride = ct_words(t + 1);
    ta.prime = ctx->d_prime;
    ta.nl = t + 2;
    ta.log_n = (int)ctx->log_n;
    int rc = launch_term_mac(ctx, s, ta, n);
    if (rc) return rc;
    const uint64_t rs_per = (uint64_t)N * (2 + 2 * (t + 1));
    if ((rc = ensure_workspace(ctx, rs_per * std::min(n, kMaxChunk)))) return rc;
    uint64_t cv[64];
    if (has_k0) consts(t, k0, cv);
    return rescale_batch(ctx, s, G, ct_words(t + 1), out, ct_words(t), n, t + 1, ctx->ws, ctx->ws_words,
                         has_k0 ? cv : nullptr, acc);
  }

  // out = (k0, 0): the trivial ciphertext of a constant
  int constant(int t, int64_t k0, uint64_t* out) {
    TermMacArgs ta;
    memset(&ta, 0, sizeof(ta));
    ta.nt = 0;
    ta.out = out;
    ta.out_bstride = ct_words(t);
    ta.prime = ctx->d_prime;
    ta.nl = t + 1;
    ta.log_n = (int)ctx->log_n;
    ta.has_add = 1;
    consts(t, k0, ta.add0);
    return launch_term_mac(ctx, s, ta, n);
  }

  // out = p(x) at level t and scale T (nc coefficients, the last nonzero)
  int eval(const double* c, int nc, int t, double T, uint64_t* out) {
    if (nc <= 1) return constant(t, nc ? rnd(c[0] * T) : 0, out);
    if (nc == 2)
      return scaled(y[0], y_stride[0], level, rnd(c[1] * T * (double)ctx->mod[t + 1] / sc[0]), t, out, nullptr,
                    true, rnd(c[0] * T));
    const int j = ceil_log2(nc), g = 1 << (j - 1);
    const int n_lo = trim_coeffs(c, g), n_hi = nc - g;
    int rc;
    const uint64_t* acc = nullptr;
    bool has_k0 = false;
    int64_t k0 = 0;
    if (n_lo >= 2) {
      if ((rc = eval(c, n_lo, t, T, out))) return rc;
      acc = out;
    } else if (n_lo == 1) {
      has_k0 = true;
      k0 = rnd(c[0] * T);
    }
    const int ly = level - (j - 1);
    if (n_hi == 1)
      return scaled(y[j - 1], y_stride[j - 1], ly, rnd(c[g] * T * (double)ctx->mod[t + 1] / sc[j - 1]), t, out, acc,
                    has_k0, k0);
    // the high part at (t+1, T q_(t+1) / s_(j-1)), times y_(j-1) at level t+1
    const int m = t + 1;
    const uint64_t hw = (uint64_t)n * ct_words(m);
    if (top + hw > cap) return set_error(CKKS_EINTERNAL, "polynomial evaluation stack exhausted");
    uint64_t* H = stack + top;
    top += hw;
    rc = eval(c + g, n_hi, m, T * (double)ctx->mod[m] / sc[j - 1], H);
    uint64_t cv[64];
    if (has_k0) consts(t, k0, cv);
    if (!rc)
      rc = mul_relin_rescale(ctx, s, H, y[j - 1], y_stride[j - 1], (uint64_t)(ly + 1) * ctx->N, rlk, out, n, m, true,
                             has_k0 ? cv : nullptr, acc);
    top -= hw;
    return rc;
  }
};

}  // namespace

int ckks_poly_eval_tree(ckks_ctx* ctx, const uint64_t* d_ct_in, int batch, int level, double scale,
                        const double* coeffs, int degree, const uint64_t* d_rlk, uint64_t* d_ct_out, double* out_scale,
                        ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_ct_in || !d_ct_out || !d_rlk || !coeffs || !out_scale || batch < 0)
    return set_error(CKKS_EINVAL, "NULL pointer or bad batch");
  if (misaligned(d_ct_in) || misaligned(d_ct_out) || misaligned(d_rlk))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (degree < 1 || degree > 64) return set_error(CKKS_ERANGE, "degree must be 1..64");
  const int depth = ceil_log2(degree + 1);
  if (level < depth) return set_error(CKKS_ERANGE, "the level must be at least ceil(log2(degree + 1))");
  if (ctx->K == 0) return set_error(CKKS_EPARAM, "relinearisation needs special primes");
  const uint32_t N = ctx->N;
  const int t = level - depth, nc = trim_coeffs(coeffs, degree + 1);
  TreeEval E;
  memset(&E, 0, sizeof(E));
  E.ctx = ctx;
  E.s = stream;
  E.rlk = d_rlk;
  E.level = level;
  E.sc[0] = scale;
  for (int j = 1; j < depth; ++j) E.sc[j] = E.sc[j - 1] * E.sc[j - 1] / (double)ctx->mod[level - j + 1];
  E.check(coeffs, nc, t, scale);
  if (E.bad) return set_error(CKKS_EINVAL, "a rounded polynomial constant reaches 2^62");
  *out_scale = scale;
  if (batch == 0) return CKKS_OK;
  const uint64_t in_ct = 2ull * (level + 1) * N, out_ct = 2ull * (t + 1) * N;
  REJECT_OVERLAP(d_ct_out, out_ct * batch, d_ct_in, in_ct * batch, "the input");
  REJECT_OVERLAP(d_ct_out, out_ct * batch, d_rlk, (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * N, "the key");
  // per item: the powers y_1 .. y_(depth-1), the constant-product scratch and
  // one high-part buffer per recursion depth
  uint64_t pw_off[8], per_item = 0;
  for (int j = 1; j < depth; ++j) {
    pw_off[j] = per_item;
    per_item += 2ull * (level - j + 1) * N;
  }
  const uint64_t g_off = per_item;
  per_item += in_ct;
  const uint64_t st_off = per_item;
  per_item += (uint64_t)depth * in_ct;
  const int chunk = (int)std::max<uint64_t>(1, std::min<uint64_t>({(uint64_t)batch, 16, (1ull << 30) / per_item}));
  if ((rc = ensure_aux(ctx, chunk * per_item))) return rc;
  uint64_t* aux = ctx->aux;
  for (int b0 = 0; b0 < batch && rc == CKKS_OK; b0 += chunk) {
    const int n = std::min(chunk, batch - b0);
    E.n = n;
    E.y[0] = d_ct_in + b0 * in_ct;
    E.y_stride[0] = in_ct;
    for (int j = 1; j < depth && rc == CKKS_OK; ++j) {
      E.y[j] = aux + chunk * pw_off[j];
      E.y_stride[j] = 2ull * (level - j + 1) * N;
      rc = mul_relin_rescale(ctx, stream, E.y[j - 1], E.y[j - 1], E.y_stride[j - 1],
                             (uint64_t)(level - j + 2) * N, d_rlk, aux + chunk * pw_off[j], n, level - j + 1, true,
                             nullptr);
    }
    if (rc) break;
    E.G = aux + chunk * g_off;
    E.stack = aux + chunk * st_off;
    E.top = 0;
    E.cap = (uint64_t)chunk * depth * in_ct;
    rc = E.eval(coeffs, nc, t, scale, d_ct_out + b0 * out_ct);
  }
  return rc;
}

int ckks_ptmatvec(ckks_ctx* ctx, const uint64_t* d_x, int n_in, const uint64_t* d_diags, int n_out, int n1, int n2,
                  const uint32_t* baby_galois, const uint64_t* const* d_evk_baby, const uint32_t* giant_galois,
                  const uint64_t* const* d_evk_giant, uint64_t* d_y, int level, unsigned flags,
                  ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_x || !d_diags || !d_y || n_in < 1 || n_out < 1 || n1 < 1 || n2 < 1)
    return set_error(CKKS_EINVAL, "NULL pointer or bad size");
  if ((n1 > 1 && (!baby_galois || !d_evk_baby)) || (n2 > 1 && (!giant_galois || !d_evk_giant)))
    return set_error(CKKS_EINVAL, "missing rotation keys");
  if (misaligned(d_x) || misaligned(d_diags) || misaligned(d_y))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  for (int b = 1; b < n1; ++b)
    if (!d_evk_baby[b - 1] || misaligned(d_evk_baby[b - 1])) return set_error(CKKS_EINVAL, "NULL or misaligned key pointer");
  for (int g = 1; g < n2; ++g)
    if (!d_evk_giant[g - 1] || misaligned(d_evk_giant[g - 1])) return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (flags & ~CKKS_NO_RESCALE) return set_error(CKKS_EINVAL, "unknown flag");
  const bool rescale = !(flags & CKKS_NO_RESCALE);
  if (rescale && level == 0) return set_error(CKKS_ERANGE, "cannot rescale at level 0");
  if (ctx->K == 0) return set_error(CKKS_EPARAM, "rotation needs special primes");
  for (int b = 1; b < n1; ++b)
    if ((rc = check_galois(ctx, baby_galois[b - 1]))) return rc;
  for (int g = 1; g < n2; ++g)
    if ((rc = check_galois(ctx, giant_galois[g - 1]))) return rc;
  const uint32_t N = ctx->N;
  const int nq = level + 1;
  const uint64_t ct = 2ull * nq * N;
  {
    const uint64_t y_words = 2ull * (rescale ? level : nq) * N * n_out;
    const uint64_t key_words = (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * N;
    REJECT_OVERLAP(d_y, y_words, d_x, ct * n_in, "the input");
    REJECT_OVERLAP(d_y, y_words, d_diags, (uint64_t)nq * N * n_out * n_in * n1 * n2, "the diagonals");
    for (int b = 1; b < n1; ++b) REJECT_OVERLAP(d_y, y_words, d_evk_baby[b - 1], key_words, "a key");
    for (int g = 1; g < n2; ++g) REJECT_OVERLAP(d_y, y_words, d_evk_giant[g - 1], key_words, "a key");
  }
  // baby [n1][n_in] ciphertexts, inner [n_out][n2], rotated [n_out][n2]: in
  // the context's operand buffer, kept between calls
  const uint64_t n_baby = ct * n1 * n_in, n_inner = ct * n_out * n2;
  if ((rc = ensure_aux(ctx, n_baby + 2 * n_inner))) return rc;
  uint64_t* baby = ctx->aux;
  uint64_t* inner = baby + n_baby;
  uint64_t* rot = inner + n_inner;
  rc = CKKS_OK;
  do {
    if (hipMemcpyAsync(baby, d_x, ct * n_in * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
      rc = set_error(CKKS_EHIP, "copy");
      break;
    }
    // baby steps: the n1-1 rotations of each input share one decomposition;
    // baby step b of input c lands at baby[b][c]
    if (n1 > 1 && (rc = rotate_hoisted(ctx, stream, d_x, ct, n_in, level, n1 - 1, baby_galois, d_evk_baby,
                                       baby + (uint64_t)n_in * ct, ct, (uint64_t)n_in * ct)))
      break;
    PtMacArgs pm;
    pm.diags = d_diags;
    pm.baby = baby;
    pm.out = inner;
    pm.prime = ctx->d_prime;
    pm.n = N;
    pm.level = level;
    pm.n_in = n_in;
    pm.n1 = n1;
    pm.n2 = n2;
    if ((rc = launch_ptmac(ctx, stream, pm, n_out))) break;
    if ((rc = rotate_giant_steps(ctx, stream, inner, rot, ct, n_out, n2, level, giant_galois, d_evk_giant))) break;
    // sum over giant steps into rot[o][0] (giant step 0 is not rotated)
    if (n2 == 1) {
      for (int o = 0; o < n_out && !rc; ++o)
        if (hipMemcpyAsync(rot + o * ct, inner + o * ct, ct * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess)
          rc = set_error(CKKS_EHIP, "copy");
    }
    for (int g = 1; g < n2 && !rc; ++g)
      rc = launch_add(ctx, stream, g == 1 ? inner : rot, rot + g * ct, rot, n_out, nq, 2, ct * n2);
    if (rc) break;
    if (rescale) {
      const uint64_t rs_per = (uint64_t)N * (2 + 2 * level);
      if ((rc = ensure_workspace(ctx, rs_per * std::min(n_out, kMaxChunk)))) break;
      rc = rescale_batch(ctx, stream, rot, ct * n2, d_y, 2ull * level * N, n_out, level, ctx->ws, ctx->ws_words);
    } else {
      for (int o = 0; o < n_out && !rc; ++o)
        if (hipMemcpyAsync(d_y + o * ct, rot + o * n2 * ct, ct * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess)
          rc = set_error(CKKS_EHIP, "copy");
    }
  } while (0);
  return rc;
}

}  // extern "C"

// Relinearisation of `batch` three-part ciphertexts T (item b at
// T + b*t_stride, [3][l+1][N]) into out (item b at out + b*out_stride,
// [2][l+1][N]): (T0, T1) + KS_{s^2 -> s}(T2), in chunks over the lanes.
static int relin_batch(Ctx* c, hipStream_t s, const uint64_t* T, uint64_t t_stride, uint64_t* out,
                       uint64_t out_stride, int batch, int level, const uint64_t* rlk) {
  const int nq = level + 1;
  const uint64_t limb = (uint64_t)nq * c->N;
  const uint64_t per = ks_ws_words(c, level);
  const int chunk = g_chunk_default();
  const int n_chunks = (batch + chunk - 1) / chunk;
  const int lanes = std::min(n_chunks, g_lanes_default());
  int rc;
  if ((rc = ensure_workspace(c, per * chunk * lanes)) || (rc = fork_lanes(c, s, lanes))) return rc;
  for (int k = 0; k < n_chunks && rc == CKKS_OK; ++k) {
    const int b0 = k * chunk, n = std::min(chunk, batch - b0);
    KSItem items[kMaxChunk];
    for (int i = 0; i < n; ++i) {
      KSItem& it = items[i];
      const uint64_t* t = T + (b0 + i) * t_stride;
      it.d = t + 2 * limb;
      it.g = 0;
      it.evk = rlk;
      it.add[0] = t;
      it.add[1] = t + limb;
      it.add_g = 0;
      it.accum = nullptr;
      it.out = out + (b0 + i) * out_stride;
    }
    rc = ks_chunk(c, lane_stream(c, s, lanes, k), level, n, items, t_stride, t_stride, 0, out_stride, nq,
                  c->ws + per * chunk * (k % lanes));
  }
  return join_lanes(c, s, lanes, rc);
}

extern "C" {

int ckks_ctmatvec(ckks_ctx* ctx, const uint64_t* d_x, int n_in, const uint64_t* d_diags, int n_out, int n1, int n2,
                  const uint64_t* d_rlk, const uint32_t* baby_galois, const uint64_t* const* d_evk_baby,
                  const uint32_t* giant_galois, const uint64_t* const* d_evk_giant, uint64_t* d_y, int level,
                  unsigned flags, ckks_stream_t stream) {
  CTX_OR_FAIL(ctx);
  if (!d_x || !d_diags || !d_rlk || !d_y || n_in < 1 || n_out < 1 || n1 < 1 || n2 < 1)
    return set_error(CKKS_EINVAL, "NULL pointer or bad size");
  if ((n1 > 1 && (!baby_galois || !d_evk_baby)) || (n2 > 1 && (!giant_galois || !d_evk_giant)))
    return set_error(CKKS_EINVAL, "missing rotation keys");
  if (misaligned(d_x) || misaligned(d_diags) || misaligned(d_rlk) || misaligned(d_y))
    return set_error(CKKS_EINVAL, "device buffers must be 16-byte aligned");
  for (int b = 1; b < n1; ++b)
    if (!d_evk_baby[b - 1] || misaligned(d_evk_baby[b - 1])) return set_error(CKKS_EINVAL, "NULL or misaligned key pointer");
  for (int g = 1; g < n2; ++g)
    if (!d_evk_giant[g - 1] || misaligned(d_evk_giant[g - 1]))
      return set_error(CKKS_EINVAL, "NULL or misaligned key pointer");
  int rc = check_level(ctx, level);
  if (rc) return rc;
  if (flags & ~CKKS_NO_RESCALE) return set_error(CKKS_EINVAL, "unknown flag");
  const bool rescale = !(flags & CKKS_NO_RESCALE);
  if (rescale && level == 0) return set_error(CKKS_ERANGE, "cannot rescale at level 0");
  if (ctx->K == 0) return set_error(CKKS_EPARAM, "relinearisation and rotation need special primes");
  for (int b = 1; b < n1; ++b)
    if ((rc = check_galois(ctx, baby_galois[b - 1]))) return rc;
  for (int g = 1; g < n2; ++g)
    if ((rc = check_galois(ctx, giant_galois[g - 1]))) return rc;
  const uint32_t N = ctx->N;
  const int nq = level + 1;
  const uint64_t ct = 2ull * nq * N, t3 = 3ull * nq * N;
  {
    const uint64_t y_words = 2ull * (rescale ? level : nq) * N * n_out;
    const uint64_t key_words = (uint64_t)ctx->dnum * 2 * (ctx->L + ctx->K) * N;
    REJECT_OVERLAP(d_y, y_words, d_x, ct * n_in, "the input");
    REJECT_OVERLAP(d_y, y_words, d_diags, ct * n_out * n_in * n1 * n2, "the diagonals");
    REJECT_OVERLAP(d_y, y_words, d_rlk, key_words, "the key");
    for (int b = 1; b < n1; ++b) REJECT_OVERLAP(d_y, y_words, d_evk_baby[b - 1], key_words, "a key");
    for (int g = 1; g < n2; ++g) REJECT_OVERLAP(d_y, y_words, d_evk_giant[g - 1], key_words, "a key");
  }
  // baby [n1][n_in] ciphertexts, tensor sums [n_out][n2] (three parts),
  // relinearised [n_out][n2], rotated [n_out][n2]: context-owned, kept
  const uint64_t n_baby = ct * n1 * n_in, n_rel = ct * n_out * n2;
  if ((rc = ensure_aux(ctx, n_baby + t3 * n_out * n2 + 2 * n_rel))) return rc;
  uint64_t* baby = ctx->aux;
  uint64_t* T = baby + n_baby;
  uint64_t* rel = T + t3 * n_out * n2;
  uint64_t* rot = rel + n_rel;
  rc = CKKS_OK;
  do {
    if (hipMemcpyAsync(baby, d_x, ct * n_in * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess) {
      rc = set_error(CKKS_EHIP, "copy");
      break;
    }
    if (n1 > 1 && (rc = rotate_hoisted(ctx, stream, d_x, ct, n_in, level, n1 - 1, baby_galois, d_evk_baby,
                                       baby + (uint64_t)n_in * ct, ct, (uint64_t)n_in * ct)))
      break;
    CtMacArgs cm;
    cm.diags = d_diags;
    cm.baby = baby;
    cm.out = T;
    cm.prime = ctx->d_prime;
    cm.n = N;
    cm.level = level;
    cm.n_in = n_in;
    cm.n1 = n1;
    cm.n2 = n2;
    if ((rc = launch_ctmac(ctx, stream, cm, n_out))) break;
    if ((rc = relin_batch(ctx, stream, T, t3, rel, ct, n_out * n2, level, d_rlk))) break;
    if ((rc = rotate_giant_steps(ctx, stream, rel, rot, ct, n_out, n2, level, giant_galois, d_evk_giant))) break;
    if (n2 == 1) {
      for (int o = 0; o < n_out && !rc; ++o)
        if (hipMemcpyAsync(rot + o * ct, rel + o * ct, ct * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess)
          rc = set_error(CKKS_EHIP, "copy");
    }
    for (int g = 1; g < n2 && !rc; ++g)
      rc = launch_add(ctx, stream, g == 1 ? rel : rot, rot + g * ct, rot, n_out, nq, 2, ct * n2);
    if (rc) break;
    if (rescale) {
      const uint64_t rs_per = (uint64_t)N * (2 + 2 * level);
      if ((rc = ensure_workspace(ctx, rs_per * std::min(n_out, kMaxChunk)))) break;
      rc = rescale_batch(ctx, stream, rot, ct * n2, d_y, 2ull * level * N, n_out, level, ctx->ws, ctx->ws_words);
    } else {
      for (int o = 0; o < n_out && !rc; ++o)
        if (hipMemcpyAsync(d_y + o * ct, rot + o * n2 * ct, ct * 8, hipMemcpyDeviceToDevice, stream) != hipSuccess)
          rc = set_error(CKKS_EHIP, "copy");
    }
  } while (0);
  return rc;
}

}  // extern "C"
