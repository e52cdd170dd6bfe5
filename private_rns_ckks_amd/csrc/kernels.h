// Argument blocks and launchers of the non-NTT kernels.  Strides are in
// 64-bit words; `*_bstride` is the distance between consecutive batch items.
#pragma once
#include "internal.h"

namespace ckks {

constexpr int kMaxChunk = 32;  // batch items per launch of the key-switch pipeline
constexpr int kMaxExt = 80;   // limbs of the extended basis: L (<= 64) + K (<= 16)

struct ModUpArgs {
  const uint64_t* x;    // y_i = x_i [qhat_i^-1]_{q_i}, coefficient form, [level+1][N] per item
  uint64_t* out;        // [beta][next][N] per item
  uint64_t x_bstride, out_bstride;
  const uint64_t* tables;
  const PrimeConst* prime;
  uint32_t n;
  int level, next, L;
  int lo[64], hi[64];
  uint64_t offset[64];
};

struct ModDownArgs {
  const uint64_t* acc;  // per item; special limb k of component c (y_k, coefficient form) at limb
                        // c*acc_comp_limbs + acc_k0 + k: [2][next][N] with (next, level+1), or [2][K][N] with (K, 0)
  uint64_t* w;          // [2][level+1][N] per item (coefficient form)
  uint64_t acc_bstride, w_bstride;
  const uint64_t* conv;   // [K][L]
  const PrimeConst* prime;
  uint32_t n;
  int level, acc_comp_limbs, acc_k0, L, K;
};

struct TensorArgs {
  const uint64_t *a, *b;  // [2][level+1][N] per item (b: component stride b_comp)
  uint64_t* out;          // [3][level+1][N] per item
  uint64_t in_bstride, out_bstride;
  uint64_t b_bstride, b_comp;  // b's item and component strides (b may hold more limbs)
  const PrimeConst* prime;
  uint32_t n;
  int level;
};

struct PtMacArgs {
  const uint64_t* diags;  // [n_out][n_in][n2][n1][level+1][N]
  const uint64_t* baby;   // [n1][n_in][2][level+1][N]
  uint64_t* out;          // [n_out][n2][2][level+1][N]
  const PrimeConst* prime;
  uint32_t n;
  int level, n_in, n1, n2;
};

struct CtMacArgs {
  const uint64_t* diags;  // [n_out][n_in][n2][n1][2][level+1][N] ciphertexts
  const uint64_t* baby;   // [n1][n_in][2][level+1][N]
  uint64_t* out;          // [n_out][n2][3][level+1][N]
  const PrimeConst* prime;
  uint32_t n;
  int level, n_in, n1, n2;
};

struct ConstMulArgs {
  const uint64_t* in;  // [2][nl][N] per item
  uint64_t* out;       // [2][nl][N] per item
  uint64_t in_bstride, out_bstride;
  const PrimeConst* prime;
  uint64_t k[64][2];  // per limb: constant mod q_i and its Shoup quotient
  int nl, log_n;
};


struct KSItem {
  const uint64_t* d;       // NTT-form input polynomial [level+1][N]
  uint32_t g;              // automorphism applied to d before switching (0 = none)
  const uint64_t* evk;     // [dnum][2][L+K][N]
  const uint64_t* add[2];  // added to output component (gathered through add_g when add_g != 0)
  uint32_t add_g;
  const uint64_t* accum;   // [2][level+1][N] added to the output, or NULL
  uint64_t* out;           // [2][out_comp_limbs][N]
};

// Key-switch workspace per item at `level` (words).
size_t ks_ws_words(const Ctx* c, int level);

// Hybrid key switch of up to kMaxChunk items whose external buffers share one
// stride (item i at base + i*stride); `ws` provides ks_ws_words per item.
int ks_chunk(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, uint64_t d_stride,
             uint64_t add_stride, uint64_t accum_stride, uint64_t out_stride, int out_comp_limbs, uint64_t* ws);

// Hoisted rotations of several inputs that share one decomposition each:
// ks_decompose raises the digits of c1 (input i at c1 + i*c1_stride, NTT form)
// to the extended basis and transforms them, into dec (input i at
// dec + i*dec_stride, ks_dec_words per input); ks_hoisted_chunk key-switches
// up to kMaxChunk rotations of ONE decomposed input (it[i].g and it[i].evk;
// the output adds it[0].add[0] gathered through it[i].add_g), using
// ks_back_words of `ws` per item.
size_t ks_dec_words(const Ctx* c, int level);
size_t ks_back_words(const Ctx* c, int level);
int ks_decompose(Ctx* c, hipStream_t s, int level, int n_in, const uint64_t* c1, uint64_t c1_stride, uint64_t* dec,
                 uint64_t dec_stride);
int ks_hoisted_chunk(Ctx* c, hipStream_t s, int level, int n_items, const KSItem* it, const uint64_t* dec,
                     const uint64_t* c1, uint64_t out_stride, uint64_t* ws);

int launch_automorph_ntt(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t* out, int npoly, int nl, uint64_t pstride,
                         uint32_t g);
int launch_automorph_coeff(Ctx* c, hipStream_t s, const uint64_t* in, uint64_t* out, int npoly, int nl,
                           uint64_t pstride, uint32_t ginv);
int launch_modup(Ctx* c, hipStream_t s, ModUpArgs& a, int beta, int batch);
int launch_moddown_conv(Ctx* c, hipStream_t s, ModDownArgs& a, int batch);
int launch_tensor(Ctx* c, hipStream_t s, TensorArgs& a, int batch);
int launch_ptmac(Ctx* c, hipStream_t s, PtMacArgs& a, int n_out);
int launch_ctmac(Ctx* c, hipStream_t s, CtMacArgs& a, int n_out);
// Rescale of `batch` items by limb `level`: v = iNTT of that limb per item
// and component ([2][N], canonical), w scratch [2][level][N], out
// [2][level][N]; add0: per-limb constant added to component 0; acc:
// [2][level][N] per item added to the output (may equal out).
int rescale_fused(Ctx* c, hipStream_t s, const uint64_t* ct, uint64_t ct_bstride, const uint64_t* v, uint64_t v_bstride,
                  uint64_t* w, uint64_t w_bstride, uint64_t* out, uint64_t out_bstride, int batch, int level,
                  const uint64_t* add0 = nullptr, const uint64_t* acc = nullptr, uint64_t acc_bstride = 0);
int launch_const_mul(Ctx* c, hipStream_t s, ConstMulArgs& a, int batch);

// Sum of constant multiples of up to kMaxTerms ciphertexts that share one
// layout: out = sum_t K_t * x_t (mod q_i, K_t signed, |K_t| < 2^62), both
// components, limbs 0 .. nl-1, plus add0[i] on component 0 when has_add; x_t
// item b at x[t] + b*x_bstride ([2][nl][N] with component stride x_comp), out
// item b at out + b*out_bstride ([2][nl][N] contiguous).  With no terms out
// is zero (plus the constant).
constexpr int kMaxTerms = 32;
struct TermMacArgs {
  const uint64_t* x[kMaxTerms];
  int64_t k[kMaxTerms];
  uint64_t add0[64];
  uint64_t* out;
  uint64_t x_bstride, x_comp, out_bstride;
  const PrimeConst* prime;
  int nt, nl, log_n, has_add;
};
int launch_term_mac(Ctx* c, hipStream_t s, TermMacArgs& a, int batch);

// Argument checks of a batched rotation (shared by the entry points that
// rotate): CKKS_OK or the error code, with the detail set.
int rotate_check(Ctx* ctx, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                 const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags);
// A checked rotation batch run entirely on stream s with the caller's
// workspace ws[ws_words] (chunks of as many items as fit, at most
// kMaxChunk): no internal streams, no allocation.
int rotate_fixed_ws(Ctx* ctx, hipStream_t s, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                    const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags, uint64_t* ws,
                    uint64_t ws_words);
// Resolves the device address of the allocation-free scratch array on the
// current device (once per device); called by context creation.
int noalloc_init_device(int device);
int launch_add(Ctx* c, hipStream_t s, const uint64_t* x, const uint64_t* y, uint64_t* out, int npoly, int nl,
               int ncomp, uint64_t bstride);

}  // namespace ckks
