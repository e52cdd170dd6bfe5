/*
 * ckks_oracle.c -- plain CPU reference ("oracle") for the RNS-CKKS rotation
 * hot path: negacyclic NTT, Galois automorphism, hybrid key switching
 * (ModUp, inner product with dnum key digits, ModDown), rotation, rescale,
 * ciphertext-ciphertext multiply with relinearisation, the baby-step /
 * giant-step matrix-vector product with plaintext or encrypted weights, and
 * polynomial evaluation.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant generator with the GPU library; the two agree only
 * because both follow the same mathematics.
 *
 * Source of the method.  The pages this work follows (the AEGIS summary on
 * gist.science, "Problem" section, challenges 2 and 3, and the
 * "Methodology" section on communication hiding) say only that the system
 * runs CKKS over a residue number system and that key switching and rotation
 * dominate Transformer matrix products and non-linear layers.  They give no
 * formula.  Every step below is therefore the standard full-RNS CKKS
 * construction with hybrid key switching, written out plainly:
 *   - Cheon, Kim, Kim, Song (2017): the CKKS scheme, rescaling by rounding;
 *   - Cheon, Han, Kim, Kim, Song (2018): the full-RNS variant;
 *   - Han, Ki (2020): hybrid key switching with dnum gadget digits;
 *   - Bajard, Eynard, Hasan, Zucca (2016): fast basis conversion;
 *   - Halevi, Shoup (2014): the diagonal / baby-step giant-step matvec.
 * The conventions that fix every output word (prime choice, root of unity,
 * NTT output order, rounding in ModUp / ModDown / rescale, key gadget) are
 * the readings listed in the design notes; each function states the one it
 * uses.
 *
 * Arithmetic is deliberately naive: every modular product is
 * (unsigned __int128)a*b % m, every sum is reduced immediately, and nothing
 * is fused, reordered or made lazy.  OpenMP only splits loops whose
 * iterations are independent (limbs, coefficients, batch items), so results
 * do not depend on the thread count.
 *
 * Layout conventions (all arrays are uint64 residues in [0, m)):
 *   limb      : N words, one residue polynomial modulo one prime;
 *   basis     : q_0..q_{L-1} (ciphertext primes) then p_0..p_{K-1};
 *   level l   : l+1 ciphertext limbs q_0..q_l;
 *   extended  : at level l, l+1+K limbs q_0..q_l, p_0..p_{K-1};
 *   ciphertext: [2][l+1][N] in NTT form, component 0 = c0, 1 = c1;
 *   switch key: [dnum][2][L+K][N] in NTT form, component 0 = b, 1 = a.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;
typedef __int128 i128;

/* ------------------------------------------------------------------ */
/* Scalar modular arithmetic                                            */
/* ------------------------------------------------------------------ */

static uint64_t mulmod(uint64_t a, uint64_t b, uint64_t m) { return (uint64_t)((u128)a * b % m); }
static uint64_t addmod(uint64_t a, uint64_t b, uint64_t m) { return (uint64_t)(((u128)a + b) % m); }
static uint64_t submod(uint64_t a, uint64_t b, uint64_t m) { return (uint64_t)(((u128)a + m - b) % m); }

static uint64_t powmod(uint64_t a, uint64_t e, uint64_t m)
{
    uint64_t r = 1 % m;
    a %= m;
    while (e) {
        if (e & 1) r = mulmod(r, a, m);
        a = mulmod(a, a, m);
        e >>= 1;
    }
    return r;
}

/* Inverse modulo a prime by Fermat's little theorem. */
static uint64_t invmod(uint64_t a, uint64_t m) { return powmod(a, m - 2, m); }

/* Signed integer reduced into [0, m). */
static uint64_t smod(i128 x, uint64_t m)
{
    i128 r = x % (i128)m;
    if (r < 0) r += m;
    return (uint64_t)r;
}

/* ------------------------------------------------------------------ */
/* Parameters: primes and roots of unity                                */
/* ------------------------------------------------------------------ */

/* Deterministic Miller-Rabin with the first twelve prime bases, which is
 * exact for every n below 3.3e24 (Sorenson and Webster, 2015). */
int orc_is_prime(uint64_t n)
{
    static const uint64_t bases[12] = {2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37};
    if (n < 2) return 0;
    for (int i = 0; i < 12; i++) {
        if (n == bases[i]) return 1;
        if (n % bases[i] == 0) return 0;
    }
    uint64_t d = n - 1;
    int s = 0;
    while ((d & 1) == 0) { d >>= 1; s++; }
    for (int i = 0; i < 12; i++) {
        uint64_t x = powmod(bases[i], d, n);
        if (x == 1 || x == n - 1) continue;
        int composite = 1;
        for (int r = 1; r < s; r++) {
            x = mulmod(x, x, n);
            if (x == n - 1) { composite = 0; break; }
        }
        if (composite) return 0;
    }
    return 1;
}

/* The `count` largest primes below 2^bits that are 1 modulo 2N, in
 * descending order.  Returns the number found. */
int orc_gen_primes(int log_n, int bits, int count, uint64_t *out)
{
    uint64_t two_n = (uint64_t)2 << log_n;
    uint64_t c = ((uint64_t)1 << bits) - two_n + 1; /* largest value < 2^bits that is 1 mod 2N */
    int found = 0;
    while (found < count && c > two_n) {
        if (orc_is_prime(c)) out[found++] = c;
        c -= two_n;
    }
    return found;
}

/* Smallest primitive 2N-th root of unity modulo the prime m (requires
 * m = 1 mod 2N).  Any x^((m-1)/2N) whose N-th power is -1 has order exactly
 * 2N; the primitive 2N-th roots are its odd powers, and the smallest of them
 * is returned.  Returns 0 if m is not 1 mod 2N. */
uint64_t orc_min_psi(uint64_t m, int log_n)
{
    uint64_t n = (uint64_t)1 << log_n, two_n = 2 * n;
    if ((m - 1) % two_n != 0) return 0;
    uint64_t r = 0;
    for (uint64_t x = 2; x < m; x++) {
        uint64_t cand = powmod(x, (m - 1) / two_n, m);
        if (powmod(cand, n, m) == m - 1) { r = cand; break; }
    }
    uint64_t r2 = mulmod(r, r, m), cur = r, best = r;
    for (uint64_t k = 0; k < n; k++) { /* cur = r^(2k+1) */
        if (cur < best) best = cur;
        cur = mulmod(cur, r2, m);
    }
    return best;
}

/* ------------------------------------------------------------------ */
/* Negacyclic NTT                                                       */
/* ------------------------------------------------------------------ */

static uint64_t bitrev(uint64_t x, int bits)
{
    uint64_t r = 0;
    for (int i = 0; i < bits; i++) { r = (r << 1) | (x & 1); x >>= 1; }
    return r;
}

/* Forward transform in place.  Output word j is the input polynomial
 * evaluated at psi^(2*brv(j)+1), i.e. the evaluations at the roots of
 * X^N + 1 in bit-reversed order.
 *
 * Method: repeated CRT splitting.  A residue modulo X^(2h) - z^2 splits into
 * residues modulo X^h - z and X^h + z by (lo + z*hi, lo - z*hi), where lo and
 * hi are the low and high halves of its coefficient vector.  X^N + 1 =
 * X^N - psi^N; at split level with `blocks` residues of size 2h, residue b
 * uses z = psi^(brv(blocks + b)) (brv over log_n bits), which keeps every
 * factor's root set equal to the odd powers assigned above. */
void orc_ntt_forward(uint64_t *a, int log_n, uint64_t m, uint64_t psi)
{
    uint64_t n = (uint64_t)1 << log_n;
    for (uint64_t blocks = 1, h = n / 2; h >= 1; blocks *= 2, h /= 2) {
        for (uint64_t b = 0; b < blocks; b++) {
            uint64_t z = powmod(psi, bitrev(blocks + b, log_n), m);
            uint64_t *lo = a + 2 * b * h, *hi = lo + h;
            for (uint64_t i = 0; i < h; i++) {
                uint64_t t = mulmod(hi[i], z, m);
                uint64_t u = lo[i];
                lo[i] = addmod(u, t, m);
                hi[i] = submod(u, t, m);
            }
        }
    }
}

/* Inverse transform in place: undoes each split in reverse order, from
 * (r1, r2) = (lo + z*hi, lo - z*hi) recovering 2*lo = r1 + r2 and
 * 2*hi = (r1 - r2) * z^-1, and divides by N at the end.  Output is natural
 * coefficient order. */
void orc_ntt_inverse(uint64_t *a, int log_n, uint64_t m, uint64_t psi)
{
    uint64_t n = (uint64_t)1 << log_n;
    uint64_t psi_inv = invmod(psi, m);
    for (uint64_t blocks = n / 2, h = 1; blocks >= 1; blocks /= 2, h *= 2) {
        for (uint64_t b = 0; b < blocks; b++) {
            uint64_t zi = powmod(psi_inv, bitrev(blocks + b, log_n), m);
            uint64_t *lo = a + 2 * b * h, *hi = lo + h;
            for (uint64_t i = 0; i < h; i++) {
                uint64_t u = lo[i], v = hi[i];
                lo[i] = addmod(u, v, m);
                hi[i] = mulmod(submod(u, v, m), zi, m);
            }
        }
    }
    uint64_t n_inv = invmod(n % m, m);
    for (uint64_t i = 0; i < n; i++) a[i] = mulmod(a[i], n_inv, m);
}

/* Batched transform over `nlimb` consecutive limbs; limb i uses modulus
 * mods[i] and root psis[i]. */
void orc_ntt_limbs(uint64_t *a, int nlimb, int log_n, const uint64_t *mods, const uint64_t *psis, int inverse)
{
    uint64_t n = (uint64_t)1 << log_n;
#pragma omp parallel for schedule(dynamic)
    for (int i = 0; i < nlimb; i++) {
        if (inverse) orc_ntt_inverse(a + (uint64_t)i * n, log_n, mods[i], psis[i]);
        else orc_ntt_forward(a + (uint64_t)i * n, log_n, mods[i], psis[i]);
    }
}

/* ------------------------------------------------------------------ */
/* Galois automorphism X -> X^g (g odd)                                  */
/* ------------------------------------------------------------------ */

/* Coefficient form: a(X^g) mod X^N + 1.  Coefficient i moves to exponent
 * i*g mod 2N; exponents in [N, 2N) wrap with a sign change since X^N = -1. */
void orc_automorph_coeff(const uint64_t *in, uint64_t *out, int nlimb, int log_n, const uint64_t *mods, uint64_t g)
{
    uint64_t n = (uint64_t)1 << log_n, two_n = 2 * n;
    for (int l = 0; l < nlimb; l++) {
        const uint64_t *x = in + (uint64_t)l * n;
        uint64_t *y = out + (uint64_t)l * n;
        uint64_t m = mods[l];
        for (uint64_t i = 0; i < n; i++) {
            uint64_t r = (uint64_t)((u128)i * g % two_n);
            if (r < n) y[r] = x[i];
            else y[r - n] = submod(0, x[i], m);
        }
    }
}

/* NTT form: word j holds a(w_j) with w_j = psi^(2brv(j)+1); the image holds
 * a(w_j^g) = a(psi^(g*(2brv(j)+1) mod 2N)), which is input word
 * brv(((g*(2brv(j)+1)) mod 2N - 1) / 2).  A pure permutation. */
void orc_automorph_ntt(const uint64_t *in, uint64_t *out, int nlimb, int log_n, uint64_t g)
{
    uint64_t n = (uint64_t)1 << log_n, two_n = 2 * n;
    for (int l = 0; l < nlimb; l++) {
        const uint64_t *x = in + (uint64_t)l * n;
        uint64_t *y = out + (uint64_t)l * n;
        for (uint64_t j = 0; j < n; j++) {
            uint64_t e = 2 * bitrev(j, log_n) + 1;
            uint64_t eg = (uint64_t)((u128)e * g % two_n);
            y[j] = x[bitrev((eg - 1) / 2, log_n)];
        }
    }
}

/* ------------------------------------------------------------------ */
/* Scheme context                                                       */
/* ------------------------------------------------------------------ */

typedef struct {
    int log_n;      /* N = 2^log_n */
    int L, K, dnum; /* ciphertext primes, special primes, gadget digits */
    const uint64_t *mod; /* [L+K]: q_0..q_{L-1}, p_0..p_{K-1} */
    const uint64_t *psi; /* [L+K] */
} orc_params;

static int alpha_of(const orc_params *P) { return (P->L + P->dnum - 1) / P->dnum; }

/* Digit j at level l covers ciphertext limbs [lo, hi). */
static void digit_range(const orc_params *P, int level, int j, int *lo, int *hi)
{
    int a = alpha_of(P);
    *lo = j * a;
    *hi = (j + 1) * a;
    if (*hi > level + 1) *hi = level + 1;
}

static int digits_at(const orc_params *P, int level)
{
    int a = alpha_of(P);
    return (level + 1 + a - 1) / a;
}

/* Modulus and root of limb t of the extended basis at level l. */
static uint64_t ext_mod(const orc_params *P, int level, int t)
{
    return t <= level ? P->mod[t] : P->mod[P->L + (t - level - 1)];
}
static uint64_t ext_psi(const orc_params *P, int level, int t)
{
    return t <= level ? P->psi[t] : P->psi[P->L + (t - level - 1)];
}
/* Key limb index of extended limb t at level l (keys carry all L+K limbs). */
static int key_limb(const orc_params *P, int level, int t)
{
    return t <= level ? t : P->L + (t - level - 1);
}

/* ------------------------------------------------------------------ */
/* Limbwise helpers                                                     */
/* ------------------------------------------------------------------ */

void orc_poly_mul(const uint64_t *a, const uint64_t *b, uint64_t *out, int nlimb, int log_n, const uint64_t *mods)
{
    uint64_t n = (uint64_t)1 << log_n;
#pragma omp parallel for
    for (int l = 0; l < nlimb; l++)
        for (uint64_t i = 0; i < n; i++) out[l * n + i] = mulmod(a[l * n + i], b[l * n + i], mods[l]);
}

void orc_poly_add(const uint64_t *a, const uint64_t *b, uint64_t *out, int nlimb, int log_n, const uint64_t *mods)
{
    uint64_t n = (uint64_t)1 << log_n;
    for (int l = 0; l < nlimb; l++)
        for (uint64_t i = 0; i < n; i++) out[l * n + i] = addmod(a[l * n + i], b[l * n + i], mods[l]);
}

void orc_poly_sub(const uint64_t *a, const uint64_t *b, uint64_t *out, int nlimb, int log_n, const uint64_t *mods)
{
    uint64_t n = (uint64_t)1 << log_n;
    for (int l = 0; l < nlimb; l++)
        for (uint64_t i = 0; i < n; i++) out[l * n + i] = submod(a[l * n + i], b[l * n + i], mods[l]);
}

/* Signed integer coefficient vector (length N) reduced into each limb. */
void orc_from_signed(const int64_t *c, uint64_t *out, int nlimb, int log_n, const uint64_t *mods)
{
    uint64_t n = (uint64_t)1 << log_n;
    for (int l = 0; l < nlimb; l++)
        for (uint64_t i = 0; i < n; i++) out[l * n + i] = smod(c[i], mods[l]);
}

/* ------------------------------------------------------------------ */
/* Basis conversion: ModUp and ModDown                                  */
/* ------------------------------------------------------------------ */

/* ModUp of digit j at level l.
 * in : the level-l polynomial in COEFFICIENT form, [l+1][N].
 * out: the digit lifted to the extended basis, COEFFICIENT form,
 *      [l+1+K][N].
 * With I the digit's limbs, Q' their product and qhat_i = Q'/q_i:
 *   y_i   = x_i * [qhat_i^-1]_{q_i} mod q_i              (unsigned, [0,q_i))
 *   out_t = sum_{i in I} y_i * [qhat_i]_{m_t} mod m_t    (t outside I)
 *   out_t = x_t                                          (t in I)
 * Unsigned (plain) fast basis conversion: out_t = X + u*Q' mod m_t for one
 * integer u in [0, |I|), X the CRT value of the digit. */
void orc_modup(const orc_params *P, int level, int j, const uint64_t *in, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int lo, hi;
    digit_range(P, level, j, &lo, &hi);
    int next = level + 1 + P->K;
    int nd = hi - lo;
    uint64_t *qhat_inv = malloc(sizeof(uint64_t) * nd);
    uint64_t *qhat_mod = malloc(sizeof(uint64_t) * nd * next);
    for (int a = 0; a < nd; a++) {
        uint64_t qi = P->mod[lo + a];
        uint64_t prod = 1;
        for (int b = 0; b < nd; b++)
            if (b != a) prod = mulmod(prod, P->mod[lo + b] % qi, qi);
        qhat_inv[a] = invmod(prod, qi);
        for (int t = 0; t < next; t++) {
            uint64_t mt = ext_mod(P, level, t);
            uint64_t pm = 1;
            for (int b = 0; b < nd; b++)
                if (b != a) pm = mulmod(pm, P->mod[lo + b] % mt, mt);
            qhat_mod[a * next + t] = pm;
        }
    }
#pragma omp parallel for
    for (int64_t c = 0; c < (int64_t)n; c++) {
        uint64_t y[64];
        for (int a = 0; a < nd; a++) y[a] = mulmod(in[(uint64_t)(lo + a) * n + c], qhat_inv[a], P->mod[lo + a]);
        for (int t = 0; t < next; t++) {
            if (t >= lo && t < hi) {
                out[(uint64_t)t * n + c] = in[(uint64_t)t * n + c];
                continue;
            }
            uint64_t mt = ext_mod(P, level, t);
            uint64_t s = 0;
            for (int a = 0; a < nd; a++) s = addmod(s, mulmod(y[a] % mt, qhat_mod[a * next + t], mt), mt);
            out[(uint64_t)t * n + c] = s;
        }
    }
    free(qhat_inv);
    free(qhat_mod);
}

/* ModDown of one extended polynomial at level l.
 * in : [l+1+K][N] in NTT form;  out: [l+1][N] in NTT form.
 * z_k = iNTT(in[p_k]); y_k = z_k * [phat_k^-1]_{p_k} mod p_k, then CENTERED:
 * ybar_k = y_k if y_k <= (p_k-1)/2 else y_k - p_k.
 * w_i = sum_k ybar_k * [phat_k]_{q_i} mod q_i;
 * out_i = (in[q_i] - NTT(w_i)) * [P^-1]_{q_i} mod q_i. */
void orc_moddown(const orc_params *P, int level, const uint64_t *in, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int K = P->K, nq = level + 1;
    const uint64_t *pm = P->mod + P->L;
    uint64_t *z = malloc(sizeof(uint64_t) * n * K);
    memcpy(z, in + (uint64_t)nq * n, sizeof(uint64_t) * n * K);
    orc_ntt_limbs(z, K, P->log_n, pm, P->psi + P->L, 1);
    uint64_t *phat_inv = malloc(sizeof(uint64_t) * K);
    uint64_t *phat_q = malloc(sizeof(uint64_t) * K * nq);
    uint64_t *pinv_q = malloc(sizeof(uint64_t) * nq);
    for (int k = 0; k < K; k++) {
        uint64_t prod = 1;
        for (int b = 0; b < K; b++)
            if (b != k) prod = mulmod(prod, pm[b] % pm[k], pm[k]);
        phat_inv[k] = invmod(prod, pm[k]);
        for (int i = 0; i < nq; i++) {
            uint64_t qi = P->mod[i], pr = 1;
            for (int b = 0; b < K; b++)
                if (b != k) pr = mulmod(pr, pm[b] % qi, qi);
            phat_q[k * nq + i] = pr;
        }
    }
    for (int i = 0; i < nq; i++) {
        uint64_t qi = P->mod[i], pr = 1;
        for (int b = 0; b < K; b++) pr = mulmod(pr, pm[b] % qi, qi);
        pinv_q[i] = invmod(pr, qi);
    }
    uint64_t *w = malloc(sizeof(uint64_t) * n * nq);
#pragma omp parallel for
    for (int64_t c = 0; c < (int64_t)n; c++) {
        i128 yb[64];
        for (int k = 0; k < K; k++) {
            uint64_t y = mulmod(z[(uint64_t)k * n + c], phat_inv[k], pm[k]);
            yb[k] = (y <= (pm[k] - 1) / 2) ? (i128)y : (i128)y - (i128)pm[k];
        }
        for (int i = 0; i < nq; i++) {
            uint64_t qi = P->mod[i], s = 0;
            for (int k = 0; k < K; k++) s = addmod(s, mulmod(smod(yb[k], qi), phat_q[k * nq + i], qi), qi);
            w[(uint64_t)i * n + c] = s;
        }
    }
    orc_ntt_limbs(w, nq, P->log_n, P->mod, P->psi, 0);
#pragma omp parallel for
    for (int i = 0; i < nq; i++) {
        uint64_t qi = P->mod[i];
        for (uint64_t c = 0; c < n; c++)
            out[(uint64_t)i * n + c] = mulmod(submod(in[(uint64_t)i * n + c], w[(uint64_t)i * n + c], qi), pinv_q[i], qi);
    }
    free(w);
    free(z);
    free(phat_inv);
    free(phat_q);
    free(pinv_q);
}

/* ------------------------------------------------------------------ */
/* Key switching, rotation                                              */
/* ------------------------------------------------------------------ */

/* Hybrid key switch of d (level l, [l+1][N], NTT form) with switching key
 * evk ([dnum][2][L+K][N], NTT form).  out = [2][l+1][N], NTT form:
 *   for each active digit j: dt_j = NTT(ModUp_j(iNTT(d)))  (extended basis)
 *   acc_b = sum_j dt_j * evk_j.b,  acc_a = sum_j dt_j * evk_j.a
 *   out = (ModDown(acc_b), ModDown(acc_a)). */
void orc_keyswitch(const orc_params *P, int level, const uint64_t *d, const uint64_t *evk, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1, next = nq + P->K, LK = P->L + P->K;
    int beta = digits_at(P, level);
    uint64_t *ext_mods = malloc(sizeof(uint64_t) * next), *ext_psis = malloc(sizeof(uint64_t) * next);
    for (int t = 0; t < next; t++) { ext_mods[t] = ext_mod(P, level, t); ext_psis[t] = ext_psi(P, level, t); }
    uint64_t *dc = malloc(sizeof(uint64_t) * n * nq);
    memcpy(dc, d, sizeof(uint64_t) * n * nq);
    orc_ntt_limbs(dc, nq, P->log_n, P->mod, P->psi, 1);
    uint64_t *acc = calloc((size_t)2 * next * n, sizeof(uint64_t));
    uint64_t *dt = malloc(sizeof(uint64_t) * n * next);
    for (int j = 0; j < beta; j++) {
        orc_modup(P, level, j, dc, dt);
        orc_ntt_limbs(dt, next, P->log_n, ext_mods, ext_psis, 0);
        for (int comp = 0; comp < 2; comp++) {
#pragma omp parallel for
            for (int t = 0; t < next; t++) {
                const uint64_t *key = evk + (((uint64_t)j * 2 + comp) * LK + key_limb(P, level, t)) * n;
                uint64_t *ac = acc + ((uint64_t)comp * next + t) * n;
                uint64_t mt = ext_mods[t];
                for (uint64_t c = 0; c < n; c++) ac[c] = addmod(ac[c], mulmod(dt[(uint64_t)t * n + c], key[c], mt), mt);
            }
        }
    }
    orc_moddown(P, level, acc, out);
    orc_moddown(P, level, acc + (uint64_t)next * n, out + (uint64_t)nq * n);
    free(acc);
    free(dt);
    free(dc);
    free(ext_mods);
    free(ext_psis);
}

#define ORC_ROT_ACCUMULATE 1u

/* Rotation by Galois element g: out = (tau_g(c0) + k0, k1) with
 * (k0, k1) = KeySwitch(tau_g(c1)) under the key for tau_g(s).  With
 * ORC_ROT_ACCUMULATE the input is added: out = ct + Rot(ct).  g = 1 gives a
 * copy (or a doubling when accumulating). */
void orc_rotate(const orc_params *P, int level, const uint64_t *ct, uint32_t g, const uint64_t *evk, uint64_t *out,
                unsigned flags)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    uint64_t *r = malloc(sizeof(uint64_t) * 2 * nq * n);
    if (g == 1) {
        memcpy(r, ct, sizeof(uint64_t) * 2 * nq * n);
    } else {
        uint64_t *t0 = malloc(sizeof(uint64_t) * nq * n), *t1 = malloc(sizeof(uint64_t) * nq * n);
        orc_automorph_ntt(ct, t0, nq, P->log_n, g);
        orc_automorph_ntt(ct + (uint64_t)nq * n, t1, nq, P->log_n, g);
        orc_keyswitch(P, level, t1, evk, r);
        orc_poly_add(r, t0, r, nq, P->log_n, P->mod);
        free(t0);
        free(t1);
    }
    if (flags & ORC_ROT_ACCUMULATE) {
        orc_poly_add(r, ct, out, nq, P->log_n, P->mod);
        orc_poly_add(r + (uint64_t)nq * n, ct + (uint64_t)nq * n, out + (uint64_t)nq * n, nq, P->log_n, P->mod);
    } else {
        memcpy(out, r, sizeof(uint64_t) * 2 * nq * n);
    }
    free(r);
}

/* Rotations of one ciphertext by n_rot Galois elements that share one basis
 * extension ("hoisting"; the AEGIS page, "Methodology", item 4, schedules
 * several rotations of the same ciphertext).  The digits of c1 are raised to
 * the extended basis and transformed once:
 *   dt_j = NTT(ModUp_j(iNTT(c1)))                       (extended basis)
 * and for every element g (out_r, [2][l+1][N]):
 *   acc_b = sum_j tau_g(dt_j) * evk_r,j.b,  acc_a = sum_j tau_g(dt_j) * evk_r,j.a
 *   out_r = (tau_g(c0) + ModDown(acc_b), ModDown(acc_a)).
 * tau_g acts on each extended limb by the NTT-form permutation.  tau_g(dt_j)
 * lifts tau_g of digit j exactly, so this is a key switch of tau_g(c1); its
 * words differ from orc_rotate's, where tau_g comes before the extension (the
 * sign changes of tau_g meet a different multiple of the digit modulus).
 * g = 1 gives a copy.  out: [n_rot][2][l+1][N]. */
void orc_rotate_hoisted(const orc_params *P, int level, const uint64_t *ct, int n_rot, const uint32_t *g,
                        const uint64_t *const *evks, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1, next = nq + P->K, LK = P->L + P->K;
    int beta = digits_at(P, level);
    uint64_t csz = (uint64_t)2 * nq * n;
    uint64_t *ext_mods = malloc(sizeof(uint64_t) * next), *ext_psis = malloc(sizeof(uint64_t) * next);
    for (int t = 0; t < next; t++) { ext_mods[t] = ext_mod(P, level, t); ext_psis[t] = ext_psi(P, level, t); }
    uint64_t *dc = malloc(sizeof(uint64_t) * n * nq);
    memcpy(dc, ct + (uint64_t)nq * n, sizeof(uint64_t) * n * nq);
    orc_ntt_limbs(dc, nq, P->log_n, P->mod, P->psi, 1);
    uint64_t *dt = malloc(sizeof(uint64_t) * n * next * beta);
    for (int j = 0; j < beta; j++) {
        orc_modup(P, level, j, dc, dt + (uint64_t)j * next * n);
        orc_ntt_limbs(dt + (uint64_t)j * next * n, next, P->log_n, ext_mods, ext_psis, 0);
    }
    uint64_t *acc = malloc(sizeof(uint64_t) * 2 * next * n);
    uint64_t *tj = malloc(sizeof(uint64_t) * next * n);
    uint64_t *t0 = malloc(sizeof(uint64_t) * nq * n);
    for (int r = 0; r < n_rot; r++) {
        uint64_t *o = out + (uint64_t)r * csz;
        if (g[r] == 1) {
            memcpy(o, ct, sizeof(uint64_t) * csz);
            continue;
        }
        memset(acc, 0, sizeof(uint64_t) * 2 * next * n);
        for (int j = 0; j < beta; j++) {
            orc_automorph_ntt(dt + (uint64_t)j * next * n, tj, next, P->log_n, g[r]);
            for (int comp = 0; comp < 2; comp++) {
#pragma omp parallel for
                for (int t = 0; t < next; t++) {
                    const uint64_t *key = evks[r] + (((uint64_t)j * 2 + comp) * LK + key_limb(P, level, t)) * n;
                    uint64_t *ac = acc + ((uint64_t)comp * next + t) * n;
                    uint64_t mt = ext_mods[t];
                    for (uint64_t c = 0; c < n; c++) ac[c] = addmod(ac[c], mulmod(tj[(uint64_t)t * n + c], key[c], mt), mt);
                }
            }
        }
        orc_moddown(P, level, acc, o);
        orc_moddown(P, level, acc + (uint64_t)next * n, o + (uint64_t)nq * n);
        orc_automorph_ntt(ct, t0, nq, P->log_n, g[r]);
        orc_poly_add(o, t0, o, nq, P->log_n, P->mod);
    }
    free(t0);
    free(tj);
    free(acc);
    free(dt);
    free(dc);
    free(ext_mods);
    free(ext_psis);
}

/* Batch of independent rotations: ct/out are [B][2][l+1][N]. */
void orc_rotate_batch(const orc_params *P, int level, const uint64_t *ct, int batch, const uint32_t *g,
                      const uint64_t *const *evks, uint64_t *out, unsigned flags)
{
    uint64_t sz = (uint64_t)2 * (level + 1) << P->log_n;
    for (int b = 0; b < batch; b++) orc_rotate(P, level, ct + b * sz, g[b], evks[b], out + b * sz, flags);
}

/* ------------------------------------------------------------------ */
/* Rescale, multiply, relinearise                                       */
/* ------------------------------------------------------------------ */

/* Rescale one polynomial from level l to l-1 (divide by q_l, rounding to
 * nearest).  v = iNTT(c[l]); vbar = v if v <= (q_l-1)/2 else v - q_l;
 * out_i = (c[i] - NTT(vbar mod q_i)) * [q_l^-1]_{q_i} mod q_i, i < l. */
static void rescale_poly(const orc_params *P, int level, const uint64_t *c, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    uint64_t ql = P->mod[level];
    uint64_t *v = malloc(sizeof(uint64_t) * n);
    memcpy(v, c + (uint64_t)level * n, sizeof(uint64_t) * n);
    orc_ntt_inverse(v, P->log_n, ql, P->psi[level]);
    uint64_t *w = malloc(sizeof(uint64_t) * n * level);
    for (int i = 0; i < level; i++) {
        uint64_t qi = P->mod[i];
        for (uint64_t k = 0; k < n; k++) {
            i128 vb = (v[k] <= (ql - 1) / 2) ? (i128)v[k] : (i128)v[k] - (i128)ql;
            w[(uint64_t)i * n + k] = smod(vb, qi);
        }
    }
    orc_ntt_limbs(w, level, P->log_n, P->mod, P->psi, 0);
#pragma omp parallel for
    for (int i = 0; i < level; i++) {
        uint64_t qi = P->mod[i], inv = invmod(ql % qi, qi);
        for (uint64_t k = 0; k < n; k++)
            out[(uint64_t)i * n + k] = mulmod(submod(c[(uint64_t)i * n + k], w[(uint64_t)i * n + k], qi), inv, qi);
    }
    free(v);
    free(w);
}

/* Rescale a ciphertext [2][l+1][N] -> [2][l][N]. */
int orc_rescale(const orc_params *P, int level, const uint64_t *ct, uint64_t *out)
{
    if (level < 1) return -2;
    uint64_t n = (uint64_t)1 << P->log_n;
    rescale_poly(P, level, ct, out);
    rescale_poly(P, level, ct + (uint64_t)(level + 1) * n, out + (uint64_t)level * n);
    return 0;
}

/* Tensor product of two ciphertexts: d0 = a0 b0, d1 = a0 b1 + a1 b0,
 * d2 = a1 b1.  out is [3][l+1][N]. */
void orc_tensor(const orc_params *P, int level, const uint64_t *a, const uint64_t *b, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    uint64_t sz = (uint64_t)nq * n;
    uint64_t *t = malloc(sizeof(uint64_t) * sz);
    orc_poly_mul(a, b, out, nq, P->log_n, P->mod);
    orc_poly_mul(a, b + sz, out + sz, nq, P->log_n, P->mod);
    orc_poly_mul(a + sz, b, t, nq, P->log_n, P->mod);
    orc_poly_add(out + sz, t, out + sz, nq, P->log_n, P->mod);
    orc_poly_mul(a + sz, b + sz, out + 2 * sz, nq, P->log_n, P->mod);
    free(t);
}

#define ORC_NO_RESCALE 2u

/* Multiply, relinearise with the key for s^2, then rescale (unless
 * ORC_NO_RESCALE).  a, b: [B][2][l+1][N]; out: [B][2][l][N] (or l+1). */
int orc_mul_relin_rescale(const orc_params *P, int level, const uint64_t *a, const uint64_t *b, const uint64_t *rlk,
                          uint64_t *out, int batch, unsigned flags)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    uint64_t sz = (uint64_t)nq * n;
    if (!(flags & ORC_NO_RESCALE) && level < 1) return -2;
    uint64_t *d = malloc(sizeof(uint64_t) * 3 * sz), *k = malloc(sizeof(uint64_t) * 2 * sz);
    for (int bi = 0; bi < batch; bi++) {
        orc_tensor(P, level, a + bi * 2 * sz, b + bi * 2 * sz, d);
        orc_keyswitch(P, level, d + 2 * sz, rlk, k);
        orc_poly_add(d, k, k, nq, P->log_n, P->mod);
        orc_poly_add(d + sz, k + sz, k + sz, nq, P->log_n, P->mod);
        if (flags & ORC_NO_RESCALE) memcpy(out + bi * 2 * sz, k, sizeof(uint64_t) * 2 * sz);
        else orc_rescale(P, level, k, out + (uint64_t)bi * 2 * level * n);
    }
    free(d);
    free(k);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Baby-step / giant-step plaintext matrix-vector product               */
/* ------------------------------------------------------------------ */

/* x: [n_in][2][l+1][N] ciphertexts.  diags: [n_out][n_in][n2][n1][l+1][N]
 * plaintexts (NTT form), where entry (o,c,g,b) already carries the inverse
 * giant-step rotation.  Baby step b (1..n1-1) rotates by Galois element
 * g_baby[b-1] with key evk_baby[b-1]; giant step g (1..n2-1) by
 * g_giant[g-1] with evk_giant[g-1].
 *   baby_{c,b} = Rot_b(x_c)                  (b = 0: x_c itself; the n1-1
 *                                             baby steps of x_c are hoisted
 *                                             rotations sharing one extension)
 *   inner_{o,g} = sum_c sum_b diag_{o,c,g,b} (*) baby_{c,b}
 *   y_o = sum_g Rot_g(inner_{o,g})           (g = 0: no rotation)
 * then y_o is rescaled unless ORC_NO_RESCALE.  y: [n_out][2][l or l+1][N].
 * Only the outputs o in [o_begin, o_end) are computed (sampling). */
int orc_ptmatvec(const orc_params *P, int level, const uint64_t *x, int n_in, const uint64_t *diags, int n_out,
                 int n1, int n2, const uint32_t *g_baby, const uint64_t *const *evk_baby, const uint32_t *g_giant,
                 const uint64_t *const *evk_giant, uint64_t *y, unsigned flags, int o_begin, int o_end)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    uint64_t sz = (uint64_t)nq * n, csz = 2 * sz;
    if (!(flags & ORC_NO_RESCALE) && level < 1) return -2;
    uint64_t *baby = malloc(sizeof(uint64_t) * csz * n_in * n1);
    for (int c = 0; c < n_in; c++) {
        memcpy(baby + (uint64_t)(c * n1) * csz, x + (uint64_t)c * csz, sizeof(uint64_t) * csz);
        if (n1 > 1)
            orc_rotate_hoisted(P, level, x + (uint64_t)c * csz, n1 - 1, g_baby, evk_baby,
                               baby + (uint64_t)(c * n1 + 1) * csz);
    }
    uint64_t *inner = malloc(sizeof(uint64_t) * csz), *acc = malloc(sizeof(uint64_t) * csz);
    uint64_t *tmp = malloc(sizeof(uint64_t) * csz), *rot = malloc(sizeof(uint64_t) * csz);
    for (int o = o_begin; o < o_end; o++) {
        memset(acc, 0, sizeof(uint64_t) * csz);
        for (int g = 0; g < n2; g++) {
            memset(inner, 0, sizeof(uint64_t) * csz);
            for (int c = 0; c < n_in; c++)
                for (int b = 0; b < n1; b++) {
                    const uint64_t *pt = diags + ((((uint64_t)o * n_in + c) * n2 + g) * n1 + b) * sz;
                    const uint64_t *ct = baby + (uint64_t)(c * n1 + b) * csz;
                    for (int comp = 0; comp < 2; comp++) {
                        orc_poly_mul(ct + comp * sz, pt, tmp + comp * sz, nq, P->log_n, P->mod);
                        orc_poly_add(inner + comp * sz, tmp + comp * sz, inner + comp * sz, nq, P->log_n, P->mod);
                    }
                }
            if (g == 0) memcpy(rot, inner, sizeof(uint64_t) * csz);
            else orc_rotate(P, level, inner, g_giant[g - 1], evk_giant[g - 1], rot, 0);
            orc_poly_add(acc, rot, acc, nq, P->log_n, P->mod);
            orc_poly_add(acc + sz, rot + sz, acc + sz, nq, P->log_n, P->mod);
        }
        if (flags & ORC_NO_RESCALE) memcpy(y + (uint64_t)o * csz, acc, sizeof(uint64_t) * csz);
        else orc_rescale(P, level, acc, y + (uint64_t)o * 2 * level * n);
    }
    free(baby);
    free(inner);
    free(acc);
    free(tmp);
    free(rot);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Baby-step / giant-step matrix-vector product with encrypted weights   */
/* ------------------------------------------------------------------ */

/* The attention output A x V of the AEGIS summary ("Methodology",
 * self-attention: the softmax weights are gathered, then multiplied with V)
 * has both operands encrypted; the pages give no packing.  Reading: the
 * diagonal method of ptmatvec with ciphertext diagonals, the tensor products
 * of one giant-step group summed before a single relinearisation (the sum of
 * tensor products is again a three-part ciphertext under 1, s, s^2):
 *   baby_{c,b}  = Rot_b(x_c)                       (hoisted, as in ptmatvec)
 *   T_{o,g}     = sum_c sum_b tensor(diag_{o,c,g,b}, baby_{c,b})
 *   R_{o,g}     = (T0 + k0, T1 + k1),  (k0, k1) = KS_{s^2 -> s}(T2)
 *   y_o         = sum_g Rot_g(R_{o,g})             (g = 0: no rotation)
 * then rescale unless ORC_NO_RESCALE.  diags: [n_out][n_in][n2][n1][2][l+1][N]
 * ciphertexts (entry (o,c,g,b) already rotated by the inverse giant step);
 * rlk: the key for s^2.  Only outputs o in [o_begin, o_end) are computed. */
int orc_ctmatvec(const orc_params *P, int level, const uint64_t *x, int n_in, const uint64_t *diags, int n_out,
                 int n1, int n2, const uint64_t *rlk, const uint32_t *g_baby, const uint64_t *const *evk_baby,
                 const uint32_t *g_giant, const uint64_t *const *evk_giant, uint64_t *y, unsigned flags,
                 int o_begin, int o_end)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    uint64_t sz = (uint64_t)nq * n, csz = 2 * sz;
    if (!(flags & ORC_NO_RESCALE) && level < 1) return -2;
    uint64_t *baby = malloc(sizeof(uint64_t) * csz * n_in * n1);
    for (int c = 0; c < n_in; c++) {
        memcpy(baby + (uint64_t)(c * n1) * csz, x + (uint64_t)c * csz, sizeof(uint64_t) * csz);
        if (n1 > 1)
            orc_rotate_hoisted(P, level, x + (uint64_t)c * csz, n1 - 1, g_baby, evk_baby,
                               baby + (uint64_t)(c * n1 + 1) * csz);
    }
    uint64_t *t = malloc(sizeof(uint64_t) * 3 * sz), *prod = malloc(sizeof(uint64_t) * 3 * sz);
    uint64_t *rel = malloc(sizeof(uint64_t) * csz), *acc = malloc(sizeof(uint64_t) * csz);
    uint64_t *rot = malloc(sizeof(uint64_t) * csz);
    for (int o = o_begin; o < o_end; o++) {
        memset(acc, 0, sizeof(uint64_t) * csz);
        for (int g = 0; g < n2; g++) {
            memset(t, 0, sizeof(uint64_t) * 3 * sz);
            for (int c = 0; c < n_in; c++)
                for (int b = 0; b < n1; b++) {
                    const uint64_t *d = diags + ((((uint64_t)o * n_in + c) * n2 + g) * n1 + b) * csz;
                    orc_tensor(P, level, d, baby + (uint64_t)(c * n1 + b) * csz, prod);
                    for (int k = 0; k < 3; k++)
                        orc_poly_add(t + k * sz, prod + k * sz, t + k * sz, nq, P->log_n, P->mod);
                }
            orc_keyswitch(P, level, t + 2 * sz, rlk, rel);
            orc_poly_add(t, rel, rel, nq, P->log_n, P->mod);
            orc_poly_add(t + sz, rel + sz, rel + sz, nq, P->log_n, P->mod);
            if (g == 0) memcpy(rot, rel, sizeof(uint64_t) * csz);
            else orc_rotate(P, level, rel, g_giant[g - 1], evk_giant[g - 1], rot, 0);
            orc_poly_add(acc, rot, acc, nq, P->log_n, P->mod);
            orc_poly_add(acc + sz, rot + sz, acc + sz, nq, P->log_n, P->mod);
        }
        if (flags & ORC_NO_RESCALE) memcpy(y + (uint64_t)o * csz, acc, sizeof(uint64_t) * csz);
        else orc_rescale(P, level, acc, y + (uint64_t)o * 2 * level * n);
    }
    free(baby);
    free(t);
    free(prod);
    free(rel);
    free(acc);
    free(rot);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Polynomial evaluation                                                 */
/* ------------------------------------------------------------------ */

/* round(x) as a signed integer, or -1 in *bad when |x| >= 2^62. */
static int64_t round_checked(double x, int *bad)
{
    if (!(fabs(x) < 4611686018427387904.0)) { *bad = 1; return 0; }
    return llround(x);
}

/* Each limb times the integer v (signed), in place: [nlimb][N]. */
static void poly_mul_int(uint64_t *a, int nlimb, int log_n, const uint64_t *mods, int64_t v)
{
    uint64_t n = (uint64_t)1 << log_n;
    for (int i = 0; i < nlimb; i++) {
        uint64_t k = smod((i128)v, mods[i]);
        for (uint64_t c = 0; c < n; c++) a[(uint64_t)i * n + c] = mulmod(a[(uint64_t)i * n + c], k, mods[i]);
    }
}

/* The constant polynomial v (signed) added in NTT form: the transform of a
 * constant is that constant in every word. */
static void poly_add_int(uint64_t *a, int nlimb, int log_n, const uint64_t *mods, int64_t v)
{
    uint64_t n = (uint64_t)1 << log_n;
    for (int i = 0; i < nlimb; i++) {
        uint64_t k = smod((i128)v, mods[i]);
        for (uint64_t c = 0; c < n; c++) a[(uint64_t)i * n + c] = addmod(a[(uint64_t)i * n + c], k, mods[i]);
    }
}

/* p(x) = sum_{k<=d} c[k] x^k on each of `batch` ciphertexts ct
 * ([batch][2][l+1][N], NTT form, scale s_x), by Horner's rule: depth d.
 *   acc = c[d] * x       every limb times K = round(c[d] * q_l), then rescale;
 *                        the scale stays s_x (the factor q_l is divided out)
 *   acc += c[d-1]        round(c[d-1] * s_acc) added to c0
 *   for k = d-2 .. 0     x' = x on acc's limbs; with l' the level of acc:
 *                        acc = rescale(relin(acc * x')), s_acc = s_acc * s_x / q_l';
 *                        acc += round(c[k] * s_acc)
 * out: [batch][2][l-d+1][N]; *out_scale the final scale.  Returns -2 when
 * level < d or d < 1, -3 when a rounded constant reaches 2^62. */
int orc_poly_eval(const orc_params *P, int level, const uint64_t *ct, int batch, double scale, const double *c,
                  int degree, const uint64_t *rlk, uint64_t *out, double *out_scale)
{
    if (degree < 1 || level < degree) return -2;
    uint64_t n = (uint64_t)1 << P->log_n;
    int d = degree, bad = 0;
    /* the constants first, so a range error leaves out untouched */
    int64_t kmul = round_checked(c[d] * (double)P->mod[level], &bad);
    int64_t kadd[64];
    double s_acc = scale;
    kadd[d - 1] = round_checked(c[d - 1] * s_acc, &bad);
    for (int k = d - 2, l = level - 1; k >= 0; k--, l--) {
        s_acc = s_acc * scale / (double)P->mod[l];
        kadd[k] = round_checked(c[k] * s_acc, &bad);
    }
    if (bad) return -3;
    uint64_t csz_in = (uint64_t)2 * (level + 1) * n;
    uint64_t *acc = malloc(sizeof(uint64_t) * csz_in), *nxt = malloc(sizeof(uint64_t) * csz_in);
    uint64_t *xd = malloc(sizeof(uint64_t) * csz_in);
    for (int b = 0; b < batch; b++) {
        const uint64_t *x = ct + b * csz_in;
        int l = level;
        memcpy(acc, x, sizeof(uint64_t) * csz_in);
        poly_mul_int(acc, l + 1, P->log_n, P->mod, kmul);
        poly_mul_int(acc + (uint64_t)(l + 1) * n, l + 1, P->log_n, P->mod, kmul);
        orc_rescale(P, l, acc, nxt);
        l--;
        memcpy(acc, nxt, sizeof(uint64_t) * 2 * (l + 1) * n);
        poly_add_int(acc, l + 1, P->log_n, P->mod, kadd[d - 1]);
        for (int k = d - 2; k >= 0; k--) {
            uint64_t lsz = (uint64_t)(l + 1) * n;
            memcpy(xd, x, sizeof(uint64_t) * lsz);
            memcpy(xd + lsz, x + (uint64_t)(level + 1) * n, sizeof(uint64_t) * lsz);
            orc_mul_relin_rescale(P, l, acc, xd, rlk, nxt, 1, 0);
            l--;
            memcpy(acc, nxt, sizeof(uint64_t) * 2 * (l + 1) * n);
            poly_add_int(acc, l + 1, P->log_n, P->mod, kadd[k]);
        }
        memcpy(out + (uint64_t)b * 2 * (l + 1) * n, acc, sizeof(uint64_t) * 2 * (l + 1) * n);
    }
    *out_scale = s_acc;
    free(acc);
    free(nxt);
    free(xd);
    return 0;
}

/* ceil(log2 k) for k >= 1 */
static int ceil_log2(int k)
{
    int r = 0;
    while ((1 << r) < k) r++;
    return r;
}

/* Depth-efficient evaluation of p(x) = sum_{k<=d} c[k] x^k (power basis) on
 * a ciphertext x ([2][l+1][N], NTT form, scale s), in E = ceil(log2(d+1))
 * levels.  Reading: the pages name polynomial approximations of GELU and the
 * softmax exponential (AEGIS summary, "Methodology" items 2-3; the Nimbus
 * post on non-linear layers) and no evaluation scheme; this is the power-basis
 * baby-step / giant-step split with every scale fixed top-down, so each
 * addition meets equal levels and scales:
 *   powers: y_0 = x; y_j = y_{j-1}^2 (multiply, relinearise, rescale) at level
 *           l - j, scale s_j = s_{j-1}^2 / q_(l-j+1);
 *   eval(c[0..n-1], target level t, target scale T), n the number of
 *   coefficients up to the last nonzero one:
 *     n = 0: zero; n = 1: the trivial ciphertext (round(c0 T), 0);
 *     n = 2: K = round(c1 T q_(t+1) / s), x's limbs 0..t+1 times K, rescaled
 *            by q_(t+1), plus round(c0 T);
 *     n > 2: j = ceil(log2 n), g = 2^(j-1); p = hi(x) * x^g + lo(x) with
 *            lo = c[0..g-1], hi = c[g..n-1]:
 *            lo is evaluated at (t, T) (two or more coefficients) or enters
 *            as the constant round(c0 T) (one);
 *            hi with one coefficient c: K = round(c T q_(t+1) / s_(j-1)),
 *            y_(j-1)'s limbs 0..t+1 times K, rescaled by q_(t+1);
 *            otherwise hi is evaluated at (t+1, T q_(t+1) / s_(j-1)), then
 *            multiplied by y_(j-1) read at its limbs 0..t+1, relinearised
 *            and rescaled by q_(t+1);
 *            the result is that term plus lo.
 *   The output is eval(c, l - E, s): level l - E, scale s.
 * Doubles are combined in the order written (left to right); rounding is
 * llround.  Evaluation order does not change any word (sums mod q). */
typedef struct {
    const orc_params *P;
    const uint64_t *rlk;
    int level;
    const uint64_t *y[8]; /* y_j: [2][level-j+1][N] */
    double s[8];
    int bad;
} tree_eval;

/* out += r, both components of [2][nl][N] */
static void ct_add(uint64_t *out, const uint64_t *r, int nl, const orc_params *P)
{
    uint64_t sz = (uint64_t)nl << P->log_n;
    orc_poly_add(out, r, out, nl, P->log_n, P->mod);
    orc_poly_add(out + sz, r + sz, out + sz, nl, P->log_n, P->mod);
}

/* out ([2][t+1][N]) += K * (y restricted to limbs 0..t+1, level ly) rescaled by q_(t+1) */
static void tree_scaled_add(const tree_eval *E, const uint64_t *y, int ly, int64_t K, int t, uint64_t *out)
{
    const orc_params *P = E->P;
    uint64_t n = (uint64_t)1 << P->log_n, m = (uint64_t)(t + 2) * n;
    uint64_t *g = malloc(sizeof(uint64_t) * 2 * m), *r = malloc(sizeof(uint64_t) * 2 * (t + 1) * n);
    memcpy(g, y, sizeof(uint64_t) * m);
    memcpy(g + m, y + (uint64_t)(ly + 1) * n, sizeof(uint64_t) * m);
    poly_mul_int(g, t + 2, P->log_n, P->mod, K);
    poly_mul_int(g + m, t + 2, P->log_n, P->mod, K);
    orc_rescale(P, t + 1, g, r);
    ct_add(out, r, t + 1, P);
    free(g);
    free(r);
}

static int tree_trim(const double *c, int n)
{
    while (n > 0 && c[n - 1] == 0.0) n--;
    return n;
}

/* The constants eval() would round, checked against 2^62 without touching
 * any ciphertext (same recursion). */
static void tree_check_node(tree_eval *E, const double *c, int n, int t, double T)
{
    const orc_params *P = E->P;
    if (n == 0) return;
    if (n <= 2) {
        if (n == 2) round_checked(c[1] * T * (double)P->mod[t + 1] / E->s[0], &E->bad);
        round_checked(c[0] * T, &E->bad);
        return;
    }
    int j = ceil_log2(n), g = 1 << (j - 1);
    int n_lo = tree_trim(c, g), n_hi = n - g;
    if (n_lo >= 2) tree_check_node(E, c, n_lo, t, T);
    else if (n_lo == 1) round_checked(c[0] * T, &E->bad);
    if (n_hi == 1) round_checked(c[g] * T * (double)P->mod[t + 1] / E->s[j - 1], &E->bad);
    else tree_check_node(E, c + g, n_hi, t + 1, T * (double)P->mod[t + 1] / E->s[j - 1]);
}

/* out = p(x) at (t, T); out is [2][t+1][N] */
static void tree_eval_node(tree_eval *E, const double *c, int n, int t, double T, uint64_t *out)
{
    const orc_params *P = E->P;
    uint64_t n_w = (uint64_t)1 << P->log_n, sz = (uint64_t)2 * (t + 1) * n_w;
    memset(out, 0, sizeof(uint64_t) * sz);
    if (n == 0) return;
    if (n <= 2) {
        if (n == 2) {
            int64_t K = round_checked(c[1] * T * (double)P->mod[t + 1] / E->s[0], &E->bad);
            tree_scaled_add(E, E->y[0], E->level, K, t, out);
        }
        poly_add_int(out, t + 1, P->log_n, P->mod, round_checked(c[0] * T, &E->bad));
        return;
    }
    int j = ceil_log2(n), g = 1 << (j - 1);
    int n_lo = tree_trim(c, g), n_hi = n - g; /* c[n-1] != 0: n_hi >= 1 */
    if (n_lo >= 2) {
        tree_eval_node(E, c, n_lo, t, T, out);
    } else if (n_lo == 1) {
        poly_add_int(out, t + 1, P->log_n, P->mod, round_checked(c[0] * T, &E->bad));
    }
    const uint64_t *yg = E->y[j - 1];
    int ly = E->level - (j - 1);
    if (n_hi == 1) {
        int64_t K = round_checked(c[g] * T * (double)P->mod[t + 1] / E->s[j - 1], &E->bad);
        tree_scaled_add(E, yg, ly, K, t, out);
        return;
    }
    /* hi at (t+1, T q_(t+1) / s_(j-1)), times y_(j-1) at level t+1 */
    int m = t + 1;
    uint64_t msz = (uint64_t)(m + 1) * n_w;
    uint64_t *h = malloc(sizeof(uint64_t) * 2 * msz), *yb = malloc(sizeof(uint64_t) * 2 * msz);
    uint64_t *prod = malloc(sizeof(uint64_t) * sz);
    tree_eval_node(E, c + g, n_hi, m, T * (double)P->mod[m] / E->s[j - 1], h);
    memcpy(yb, yg, sizeof(uint64_t) * msz);
    memcpy(yb + msz, yg + (uint64_t)(ly + 1) * n_w, sizeof(uint64_t) * msz);
    orc_mul_relin_rescale(P, m, h, yb, E->rlk, prod, 1, 0);
    ct_add(out, prod, t + 1, P);
    free(h);
    free(yb);
    free(prod);
}

/* Returns -2 if degree < 1, degree > 64 or level < ceil(log2(degree+1)),
 * -3 if a constant reaches 2^62 (nothing written).  out: [batch][2][l-E+1][N]. */
int orc_poly_eval_tree(const orc_params *P, int level, const uint64_t *ct, int batch, double scale, const double *c,
                       int degree, const uint64_t *rlk, uint64_t *out, double *out_scale)
{
    int d = degree;
    if (d < 1 || d > 64) return -2;
    int depth = ceil_log2(d + 1);
    if (level < depth) return -2;
    uint64_t n = (uint64_t)1 << P->log_n;
    int t = level - depth;
    uint64_t osz = (uint64_t)2 * (t + 1) * n;
    tree_eval E;
    memset(&E, 0, sizeof(E));
    E.P = P;
    E.rlk = rlk;
    E.level = level;
    uint64_t *pw[8] = {0};
    E.s[0] = scale;
    for (int j = 1; j < depth; j++) E.s[j] = E.s[j - 1] * E.s[j - 1] / (double)P->mod[level - j + 1];
    int nc = tree_trim(c, d + 1);
    tree_check_node(&E, c, nc, t, scale);
    if (E.bad) return -3;
    for (int bi = 0; bi < batch; bi++) {
        const uint64_t *x = ct + (uint64_t)bi * 2 * (level + 1) * n;
        E.y[0] = x;
        for (int j = 1; j < depth; j++) {
            int lp = level - j + 1; /* level of y_(j-1) */
            if (!pw[j]) pw[j] = malloc(sizeof(uint64_t) * 2 * (level - j + 1) * n);
            orc_mul_relin_rescale(P, lp, E.y[j - 1], E.y[j - 1], rlk, pw[j], 1, 0);
            E.y[j] = pw[j];
        }
        tree_eval_node(&E, c, nc, t, scale, out + (uint64_t)bi * osz);
    }
    for (int j = 1; j < depth; j++) free(pw[j]);
    *out_scale = scale;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Keys, encryption, decryption (host-side set-up and checking)          */
/* ------------------------------------------------------------------ */

/* Secret key s (ternary coefficients) in NTT form on all L+K limbs. */
void orc_secret_ntt(const orc_params *P, const int8_t *s, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int LK = P->L + P->K;
    int64_t *c = malloc(sizeof(int64_t) * n);
    for (uint64_t i = 0; i < n; i++) c[i] = s[i];
    orc_from_signed(c, out, LK, P->log_n, P->mod);
    orc_ntt_limbs(out, LK, P->log_n, P->mod, P->psi, 0);
    free(c);
}

/* Switching key from s_from to s (both NTT form, L+K limbs):
 * for digit j < dnum with limb set D_j:
 *   evk_j.a = a_j (uniform, given in NTT form),
 *   evk_j.b = -a_j*s + e_j + [P]_{m_t} * s_from   on limbs t in D_j,
 *   evk_j.b = -a_j*s + e_j                        elsewhere,
 * where P is the product of the special primes (raw-residue gadget).
 * a: [dnum][L+K][N] uniform; e: [dnum][N] signed error coefficients. */
void orc_make_switch_key(const orc_params *P, const uint64_t *s_from, const uint64_t *s, const uint64_t *a,
                         const int64_t *e, uint64_t *evk)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int LK = P->L + P->K, alpha = alpha_of(P);
    uint64_t *et = malloc(sizeof(uint64_t) * n * LK);
    for (int j = 0; j < P->dnum; j++) {
        orc_from_signed(e + (uint64_t)j * n, et, LK, P->log_n, P->mod);
        orc_ntt_limbs(et, LK, P->log_n, P->mod, P->psi, 0);
        for (int t = 0; t < LK; t++) {
            uint64_t m = P->mod[t];
            uint64_t pmod = 1;
            for (int k = 0; k < P->K; k++) pmod = mulmod(pmod, P->mod[P->L + k] % m, m);
            int in_digit = (t < P->L) && (t >= j * alpha) && (t < (j + 1) * alpha);
            const uint64_t *aj = a + ((uint64_t)j * LK + t) * n;
            uint64_t *kb = evk + (((uint64_t)j * 2 + 0) * LK + t) * n;
            uint64_t *ka = evk + (((uint64_t)j * 2 + 1) * LK + t) * n;
            for (uint64_t c = 0; c < n; c++) {
                uint64_t v = submod(et[(uint64_t)t * n + c], mulmod(aj[c], s[(uint64_t)t * n + c], m), m);
                if (in_digit) v = addmod(v, mulmod(pmod, s_from[(uint64_t)t * n + c], m), m);
                kb[c] = v;
                ka[c] = aj[c];
            }
        }
    }
    free(et);
}

/* Symmetric encryption at level l of a plaintext pt ([l+1][N], NTT form):
 * c1 = a (uniform, NTT form), c0 = -a*s + NTT(e) + pt. */
void orc_encrypt(const orc_params *P, int level, const uint64_t *pt, const uint64_t *s, const uint64_t *a,
                 const int64_t *e, uint64_t *ct)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    uint64_t *et = malloc(sizeof(uint64_t) * n * nq);
    orc_from_signed(e, et, nq, P->log_n, P->mod);
    orc_ntt_limbs(et, nq, P->log_n, P->mod, P->psi, 0);
    for (int t = 0; t < nq; t++) {
        uint64_t m = P->mod[t];
        for (uint64_t c = 0; c < n; c++) {
            uint64_t i = (uint64_t)t * n + c;
            uint64_t v = submod(et[i], mulmod(a[i], s[i], m), m);
            ct[i] = addmod(v, pt[i], m);
            ct[(uint64_t)nq * n + i] = a[i];
        }
    }
    free(et);
}

/* Decryption to coefficient form: iNTT(c0 + c1*s), [l+1][N]. */
void orc_decrypt_coeff(const orc_params *P, int level, const uint64_t *ct, const uint64_t *s, uint64_t *out)
{
    uint64_t n = (uint64_t)1 << P->log_n;
    int nq = level + 1;
    for (int t = 0; t < nq; t++) {
        uint64_t m = P->mod[t];
        for (uint64_t c = 0; c < n; c++) {
            uint64_t i = (uint64_t)t * n + c;
            out[i] = addmod(ct[i], mulmod(ct[(uint64_t)nq * n + i], s[i], m), m);
        }
    }
    orc_ntt_limbs(out, nq, P->log_n, P->mod, P->psi, 1);
}

/* Number of OpenMP threads the batched loops use (for reporting). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
void orc_set_num_threads(int n) { omp_set_num_threads(n); }
#else
int orc_num_threads(void) { return 1; }
void orc_set_num_threads(int n) { (void)n; }
#endif
