/*
 * ckks.h -- C ABI of the MI355X (gfx950) RNS-CKKS rotation hot-path library
 * (libckks_mi355x.so).
 *
 * What it computes.  The AEGIS pages on gist.science ("Problem" section,
 * challenges 2 and 3; "Methodology", communication hiding) state that
 * encrypted Transformer inference runs CKKS over a residue number system and
 * that key switching and rotation, needed by every matrix product and
 * non-linear layer, dominate the work; the FFN layer does local polynomial
 * multiplication and attention computes Q x K^T ("Methodology", items 2 and
 * 3).  The pages give no formula, so every call follows the standard full-RNS
 * CKKS construction with hybrid key switching (Cheon-Kim-Kim-Song 2017;
 * Cheon-Han-Kim-Kim-Song 2018; Han-Ki 2020; fast basis conversion of
 * Bajard-Eynard-Hasan-Zucca 2016; diagonal matvec of Halevi-Shoup 2014).
 *
 * Conventions shared by every call
 *   Words      uint64, one residue per word, fully reduced to [0, m) on entry
 *              and on exit.  Inputs with a word >= its modulus are undefined.
 *   Basis      q_0 .. q_{L-1} (ciphertext primes), then p_0 .. p_{K-1}
 *              (special primes).  A level-l polynomial holds limbs q_0..q_l.
 *   Limb       N consecutive words (one residue polynomial); arrays are
 *              limb-major: [..][limb][N].
 *   NTT form   word j of a limb is the polynomial evaluated at
 *              psi^(2*brv(j)+1) (bit-reversed evaluation order), psi the
 *              limb's 2N-th root of unity (by default the smallest primitive
 *              one).  Ciphertexts, keys and plaintexts are in NTT form.
 *   Ciphertext [2][l+1][N]: component 0 = c0, component 1 = c1; decryption
 *              is c0 + c1*s.
 *   Switch key [dnum][2][L+K][N]: digit j, component 0 = b, 1 = a, with
 *              b_j + a_j*s = e_j + [P]_{m_t} * s' on the limbs t of digit j
 *              (digit j = q_{j*alpha} .. q_{(j+1)*alpha-1}, alpha =
 *              ceil(L/dnum)) and b_j + a_j*s = e_j elsewhere; P = prod p_k.
 *              At level l the same key is used with limbs l+1..L-1 skipped.
 *   Galois     elements are odd integers in [1, 2N); X -> X^g.  The library
 *              has no slot convention: a left rotation by k slots in the
 *              usual encoding is g = 5^k mod 2N.
 *   Memory     d_* arguments are device pointers (HIP), owned by the caller,
 *              not retained after the call's stream work completes, each
 *              16-byte aligned (CKKS_EINVAL otherwise; hipMalloc gives 256).
 *              Host arrays (galois element lists, key pointer lists) are
 *              read before the call returns.
 *   Streams    every compute call enqueues on `stream` and returns; outputs
 *              are valid after the stream is synchronised.  A context is not
 *              thread-safe: use one context per host thread / stream.
 *   Aliasing   ckks_ntt works in place; every other call requires its
 *              outputs not to overlap its inputs.
 *   Errors     every call returns CKKS_OK (0) or a negative CKKS_E* code; a
 *              detail string is kept per host thread (ckks_last_error).  No
 *              C++ exception crosses this interface.  On error no output is
 *              written unless the code is CKKS_EHIP (a failed launch may
 *              leave outputs partially written).
 */
#ifndef CKKS_MI355X_H
#define CKKS_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* ckks_stream_t; /* a hipStream_t; NULL = the null stream */

enum {
  CKKS_OK = 0,
  CKKS_EINVAL = -1,    /* null or misaligned pointer, bad count, even or out-of-range Galois element */
  CKKS_ERANGE = -2,    /* level out of range, rescale at level 0, limb range outside the basis */
  CKKS_ENOMEM = -3,    /* device or host allocation failed */
  CKKS_EHIP = -4,      /* HIP launch or API failure */
  CKKS_EPARAM = -5,    /* invalid parameter set */
  CKKS_EINTERNAL = -6  /* internal error */
};

/* flags */
#define CKKS_ROT_ACCUMULATE 1u /* ckks_rotate: out = in + Rot(in) */
#define CKKS_NO_RESCALE 2u     /* ckks_mul_relin_rescale / ckks_ptmatvec: keep level l */

typedef struct ckks_ctx ckks_ctx;

typedef struct {
  uint32_t log_n;      /* N = 2^log_n, 10 <= log_n <= 16 */
  uint32_t n_q;        /* L: ciphertext primes, 1..64 */
  uint32_t n_p;        /* K: special primes, 0..16; when K > 0, K == ceil(L/dnum) */
  uint32_t dnum;       /* gadget digits, 1..L; when K > 0, ceil(L/dnum) <= 16 */
  const uint64_t* q;   /* host [n_q]: distinct primes, each = 1 mod 2N, < 2^62 */
  const uint64_t* p;   /* host [n_p]: distinct primes, each = 1 mod 2N, < 2^62 */
  const uint64_t* psi; /* host [n_q+n_p] primitive 2N-th roots, or NULL = smallest ones */
} ckks_params;

/* ---- host-only set-up (no GPU needed) ---------------------------------- */

/* The `count` largest primes below 2^bits that are 1 mod 2^(log_n+1), in
 * descending order, written to out[count] (host).  bits in [log_n+2, 62].
 * Parameter set-up for the benchmark parameter reading (largest NTT-friendly
 * primes); CKKS_EPARAM if fewer exist. */
int ckks_find_primes(uint32_t log_n, uint32_t bits, uint32_t count, uint64_t* out);

/* Checks a parameter set: sizes, primality (deterministic Miller-Rabin),
 * q = 1 mod 2N, distinctness, the K == ceil(L/dnum) rule and, when given,
 * that each psi is a primitive 2N-th root.  Returns CKKS_OK or CKKS_EPARAM. */
int ckks_params_validate(const ckks_params* params);

const char* ckks_strerror(int status);
const char* ckks_last_error(void); /* detail of this thread's last failure ("" if none) */

/* ---- context ------------------------------------------------------------- */

/* Validates params, selects HIP device `hip_device`, and uploads the
 * per-prime twiddle tables and basis-conversion constants.  *out owns that
 * device memory plus a workspace grown on demand. */
int ckks_ctx_create(const ckks_params* params, int hip_device, ckks_ctx** out);
int ckks_ctx_destroy(ckks_ctx* ctx);
/* The roots in use (n_q+n_p values, host). */
int ckks_ctx_psi(const ckks_ctx* ctx, uint64_t* out);

/* ---- kernel timing trace (profiling aid) ------------------------------------ */

typedef struct {
  int32_t launches;  /* traced launches since ckks_trace_begin */
  double total_ms;   /* sum of their durations (HIP events on the launch stream) */
  double work_units; /* algorithmic work of those launches, in 64-bit modmul-class
                        operations: one NTT butterfly, one 64x64-bit multiply-
                        accumulate, one modular reduction or one constant
                        multiplication each count 1 */
} ckks_trace_stats;

/* Start tracing the kernel family `kernel`: every later launch of it on any
 * stream is bracketed by a HIP event pair on that stream.  Families:
 * "ntt_pass" (plain NTT / inverse NTT passes), the key switch's fused
 * passes "intt_row_gather" (automorphism gather + inverse row pass),
 * "ip_special" (forward row pass + key inner product on the special limbs +
 * inverse row pass of the accumulators), "comb_ip" (forward row pass + key
 * inner product on the ciphertext limbs + final combination) and
 * "ntt_row_combine" (forward row pass + final combination, hoisted
 * rotations), "automorph", "modup",
 * "moddown_conv", "rescale", "tensor", "ptmac", "ctmac", "add",
 * "const_mul", "term_mac" (polynomial evaluation's constant multiples),
 * "ip_gather".  NULL or "" stops tracing.
 * Tracing adds two event records per traced launch and nothing else. */
int ckks_trace_begin(ckks_ctx* ctx, const char* kernel);
/* Waits for the recorded events, returns the totals and stops tracing. */
int ckks_trace_end(ckks_ctx* ctx, ckks_trace_stats* out);

/* ---- hot path ------------------------------------------------------------ */

/* Source: AEGIS summary (gist.science), "Problem", challenge 2: ciphertexts
 * live as RNS residue polynomials (one per modulus of the chain) and the
 * matrix products and non-linear layers run key switching and rotation on
 * them; the negacyclic NTT per residue polynomial is the transform every one
 * of those operations is built on (the pages name no transform; standard
 * full-RNS CKKS).
 * Negacyclic NTT (inverse = 0) or inverse NTT with the 1/N factor
 * (inverse = 1), in place, on d_data = [npoly][n_limb][N]; limb i of every
 * polynomial uses basis prime limb_begin + i.  Forward maps coefficient form
 * to NTT form (bit-reversed evaluation order), inverse maps back.
 * CKKS_ERANGE if limb_begin + n_limb exceeds L+K. */
int ckks_ntt(ckks_ctx* ctx, uint64_t* d_data, int npoly, int limb_begin, int n_limb, int inverse,
             ckks_stream_t stream);

/* Source: AEGIS summary, "Problem", challenge 2 (rotations are frequent in
 * the matrix products and non-linear layers) and "Methodology", item 4
 * (rotations by several offsets, reordered); the automorphism X -> X^g is the
 * slot permutation of a rotation.
 * Galois automorphism X -> X^g on d_in = [npoly][level+1][N] (limbs
 * q_0..q_level) into d_out (same shape).  domain 0: NTT form (a permutation
 * of words); domain 1: coefficient form (a signed permutation). */
int ckks_automorph(ckks_ctx* ctx, const uint64_t* d_in, uint64_t* d_out, int npoly, int level, uint32_t galois_elt,
                   int domain, ckks_stream_t stream);

/* Source: AEGIS summary, "Problem", challenge 2 (key switching is needed by
 * every matrix product and non-linear layer and couples all RNS components)
 * and "Methodology", item 1 (the components that take part in one key switch
 * are kept together on one device: the whole switch runs in one place, as
 * here).
 * Hybrid key switch of d_poly ([level+1][N], NTT form) with the switch key
 * d_evk ([dnum][2][L+K][N]) into d_out ([2][level+1][N], NTT form):
 * per active digit, ModUp (unsigned fast basis conversion to the other limbs
 * and the special primes), NTT, inner product with the key digit, then
 * ModDown (centered conversion of the special part, multiply by P^-1).
 * Requires K > 0. */
int ckks_keyswitch(ckks_ctx* ctx, const uint64_t* d_poly, const uint64_t* d_evk, uint64_t* d_out, int level,
                   ckks_stream_t stream);

/* Source: AEGIS summary, "Problem", challenge 2 (rotation with key
 * switching in every matrix product and non-linear layer) and
 * "Methodology", item 4 (several rotations with different offsets in flight
 * at once: here a batch, one offset and key per ciphertext).
 * Batched homomorphic rotation: for b < batch, ciphertext b of d_ct_in
 * ([batch][2][level+1][N]) is mapped by Galois element galois_elts[b]
 * (host array) and key-switched back with the switch key d_evks[b] (host
 * array of device pointers, each [dnum][2][L+K][N], the key for
 * tau_g(s) -> s): out = (tau_g(c0) + k0, k1), (k0, k1) = KS(tau_g(c1)).
 * galois element 1 is the identity (copy, no key read; its key pointer may
 * be NULL).  With CKKS_ROT_ACCUMULATE, out = in + Rot(in). */
int ckks_rotate(ckks_ctx* ctx, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags, ckks_stream_t stream);

/* Allocation-free variant of ckks_rotate, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, checks and output words as
 * ckks_rotate; the difference is where the key-switch workspace comes from
 * and where the work runs:
 *   - the workspace is a library-owned device array of
 *     CKKS_NOALLOC_SCRATCH_BYTES per GPU (held from the first context
 *     created on that GPU until the process ends), not a buffer grown with
 *     hipMalloc; the call makes no allocation of any kind (device, host
 *     pinned, streams or events; kernel tracing is off for it);
 *   - every kernel runs on `stream` in order, in chunks of as many
 *     ciphertexts as the scratch holds (no internal streams).
 * CKKS_ERANGE if one ciphertext's workspace at `level` exceeds the scratch
 * (at N = 2^16 with 24 + 8 primes and dnum = 3 one ciphertext at level 23
 * takes 92 MiB: N x (24 + 3 x 32 + 2 x 8 + 2 x 24) words).  All calls on one GPU share that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * wrong words.  Nothing in the scratch needs clearing between calls. */
#define CKKS_NOALLOC_SCRATCH_BYTES (128ull << 20)
int ckks_rotate_noalloc(ckks_ctx* ctx, const uint64_t* d_ct_in, uint64_t* d_ct_out, int batch, int level,
                        const uint32_t* galois_elts, const uint64_t* const* d_evks, unsigned flags,
                        ckks_stream_t stream);

/* Hoisted rotations (AEGIS page, "Methodology", item 4: several rotations of
 * one ciphertext): each of the n_in ciphertexts of d_ct_in
 * ([n_in][2][level+1][N]) is rotated by every galois_elts[r] (host array,
 * r < n_rot) with the switch key d_evks[r] (host array of device pointers)
 * into d_ct_out ([n_in][n_rot][2][level+1][N]).  The digits of c1 are raised
 * to the extended basis and transformed once per ciphertext; each rotation
 * then applies tau_g to those extended limbs (an NTT-form permutation) before
 * the inner product, so out = (tau_g(c0) + k0, k1) with (k0, k1) the key
 * switch of tau_g(c1) whose decomposition is tau_g of c1's.  The result
 * decrypts like ckks_rotate's but its words differ: the automorphism's sign
 * changes meet the raised digit rather than the digit.  Galois element 1 is
 * a copy (its key pointer may be NULL).  Requires K > 0. */
int ckks_rotate_hoisted(ckks_ctx* ctx, const uint64_t* d_ct_in, int n_in, int level, int n_rot,
                        const uint32_t* galois_elts, const uint64_t* const* d_evks, uint64_t* d_ct_out,
                        ckks_stream_t stream);

/* Rescale (divide by q_level, rounding to nearest) of d_in
 * ([batch][2][level+1][N]) into d_out ([batch][2][level][N]).
 * CKKS_ERANGE at level 0. */
int ckks_rescale(ckks_ctx* ctx, const uint64_t* d_in, uint64_t* d_out, int batch, int level, ckks_stream_t stream);

/* Source: AEGIS summary, "Methodology", item 3 (self-attention: the product
 * Q x K^T of two encrypted operands, followed by a polynomial softmax, which
 * needs the product relinearised and rescaled).
 * Batched ciphertext product: tensor (d0 = a0 b0, d1 = a0 b1 + a1 b0,
 * d2 = a1 b1), relinearisation with d_rlk (switch key s^2 -> s):
 * (d0, d1) + KS(d2), then rescale.  d_a, d_b: [batch][2][level+1][N];
 * d_out: [batch][2][level][N], or [batch][2][level+1][N] with
 * CKKS_NO_RESCALE.  Requires K > 0; CKKS_ERANGE when rescaling at level 0. */
int ckks_mul_relin_rescale(ckks_ctx* ctx, const uint64_t* d_a, const uint64_t* d_b, const uint64_t* d_rlk,
                           uint64_t* d_out, int batch, int level, unsigned flags, ckks_stream_t stream);

/* Polynomial p(x) = sum_{k<=degree} coeffs[k] x^k (host doubles) on each of
 * the batch ciphertexts d_ct_in ([batch][2][level+1][N], NTT form, scale
 * `scale`), by Horner's rule (the polynomial approximations of the nonlinear
 * layers, AEGIS page "Methodology" and the Nimbus post; no scheme is given):
 *   acc = c_d * x         every limb times K = round(c_d * q_level), rescale
 *                         (the scale stays `scale`)
 *   acc += c_{d-1}        round(c_{d-1} * s_acc) added to c0 in NTT form
 *   for k = d-2 .. 0      acc = rescale(relin(acc * x)) with x restricted to
 *                         acc's limbs, s_acc = s_acc * scale / q_l (l the
 *                         level of acc before the product); acc += c_k
 * Rounding is llround; the constants must stay below 2^62 (CKKS_EINVAL).
 * d_ct_out: [batch][2][level-degree+1][N]; *out_scale receives the output
 * scale.  Needs 1 <= degree <= level and K > 0 (d_rlk: the s^2 -> s key).
 * The scale should be close to the primes so the rescales keep it. */
int ckks_poly_eval(ckks_ctx* ctx, const uint64_t* d_ct_in, int batch, int level, double scale, const double* coeffs,
                   int degree, const uint64_t* d_rlk, uint64_t* d_ct_out, double* out_scale, ckks_stream_t stream);

/* Source: AEGIS summary, "Methodology", items 2-3 (the nonlinear layers,
 * GELU and the softmax exponential, evaluated locally as polynomial
 * approximations) and the Nimbus post on non-linear layers (the exponential's
 * inputs concentrate on [-4, 0]); neither fixes an evaluation scheme.
 * Polynomial p(x) = sum_{k<=degree} coeffs[k] x^k (host doubles, power
 * basis) in E = ceil(log2(degree + 1)) levels (Horner's takes degree), by the
 * baby-step / giant-step split with every scale fixed top-down:
 *   powers y_0 = x, y_j = y_(j-1)^2 (multiply, relinearise with d_rlk,
 *   rescale): level l - j, scale s_j = s_(j-1)^2 / q_(l-j+1);
 *   eval(c[0..n-1], level t, scale T), n counting up to the last nonzero
 *   coefficient:
 *     n <= 1: the trivial ciphertext (llround(c0 T), 0);
 *     n = 2:  x's limbs 0..t+1 times K = llround(c1 T q_(t+1) / s), rescaled
 *             by q_(t+1), plus llround(c0 T);
 *     n > 2:  g = 2^(ceil(log2 n) - 1), p = hi(x) y_j + lo(x) with
 *             y_j = x^g, lo = c[0..g-1], hi = c[g..n-1]; lo is evaluated at
 *             (t, T) (or is the constant llround(c0 T)); a one-coefficient hi
 *             multiplies y_j's limbs 0..t+1 by llround(c T q_(t+1) / s_j) and
 *             rescales; otherwise hi is evaluated at (t+1, T q_(t+1) / s_j),
 *             multiplied by y_j at level t+1, relinearised and rescaled;
 *   output = eval(c, l - E, scale): level l - E, scale `scale`.
 * Doubles combine left to right as written; zero coefficients cost nothing.
 * d_ct_in: [batch][2][level+1][N], NTT form; d_ct_out:
 * [batch][2][level - E + 1][N].  CKKS_ERANGE unless 1 <= degree <= 64 and
 * level >= E; CKKS_EINVAL when a constant reaches 2^62 (checked before any
 * work is enqueued).  Needs K > 0.  The powers and intermediates live in a
 * context-owned buffer grown on demand (growing it synchronises the device);
 * otherwise the call only enqueues work on `stream`. */
int ckks_poly_eval_tree(ckks_ctx* ctx, const uint64_t* d_ct_in, int batch, int level, double scale,
                        const double* coeffs, int degree, const uint64_t* d_rlk, uint64_t* d_ct_out,
                        double* out_scale, ckks_stream_t stream);

/* Source: AEGIS summary, "Methodology", item 2 (FFN: each device multiplies
 * its encrypted activations by the weight slices of one output group, locally,
 * as polynomial products); the diagonal (BSGS) method is the standard way to
 * run that product on packed slots (Halevi-Shoup 2014).
 * Baby-step / giant-step ciphertext x plaintext matrix-vector product.
 *   d_x      [n_in][2][level+1][N] input ciphertexts
 *   d_diags  [n_out][n_in][n2][n1][level+1][N] plaintexts (NTT form); entry
 *            (o, c, g, b) is the diagonal for offset n1*g + b, already
 *            rotated by the inverse of giant step g
 *   baby     n1-1 Galois elements / switch keys for the baby steps 1..n1-1
 *   giant    n2-1 Galois elements / switch keys for the giant steps 1..n2-1
 *   d_y      [n_out][2][level][N] (level+1 with CKKS_NO_RESCALE)
 * y_o = sum_g Rot_g( sum_c sum_b diag(o,c,g,b) * Rot_b(x_c) ), then rescale.
 * The baby-step rotations are computed once and shared by all outputs, as
 * hoisted rotations of each input (ckks_rotate_hoisted).  The intermediate
 * ciphertexts live in a context-owned buffer grown on demand (growing it
 * synchronises the device); otherwise the call only enqueues work. */
int ckks_ptmatvec(ckks_ctx* ctx, const uint64_t* d_x, int n_in, const uint64_t* d_diags, int n_out, int n1, int n2,
                  const uint32_t* baby_galois, const uint64_t* const* d_evk_baby, const uint32_t* giant_galois,
                  const uint64_t* const* d_evk_giant, uint64_t* d_y, int level, unsigned flags,
                  ckks_stream_t stream);

/* Baby-step / giant-step matrix-vector product with encrypted weights: the
 * attention output A x V, where the softmax weights A arrive encrypted
 * (AEGIS page, "Methodology", self-attention: the weights are gathered and
 * multiplied with V; no packing is given, so this is the diagonal method of
 * ckks_ptmatvec with ciphertext diagonals).
 *   d_x      [n_in][2][level+1][N] input ciphertexts (V)
 *   d_diags  [n_out][n_in][n2][n1][2][level+1][N] ciphertexts (A's
 *            diagonals); entry (o, c, g, b) is the diagonal for offset
 *            n1*g + b, already rotated by the inverse of giant step g
 *   d_rlk    [dnum][2][L+K][N] switching key for s^2
 *   baby / giant  Galois elements and keys as in ckks_ptmatvec
 *   d_y      [n_out][2][level][N] (level+1 with CKKS_NO_RESCALE)
 * T_og = sum_c sum_b tensor(diag(o,c,g,b), Rot_b(x_c)) (three parts, summed
 * before one relinearisation per (o, g)); y_o = sum_g Rot_g(relin(T_og)),
 * then rescale.  Buffers and errors as in ckks_ptmatvec; K > 0. */
int ckks_ctmatvec(ckks_ctx* ctx, const uint64_t* d_x, int n_in, const uint64_t* d_diags, int n_out, int n1, int n2,
                  const uint64_t* d_rlk, const uint32_t* baby_galois, const uint64_t* const* d_evk_baby,
                  const uint32_t* giant_galois, const uint64_t* const* d_evk_giant, uint64_t* d_y, int level,
                  unsigned flags, ckks_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CKKS_MI355X_H */
