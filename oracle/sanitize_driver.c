/*
 * sanitize_driver.c -- runs every oracle entry point once on small random
 * inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (the oracle is test infrastructure; this driver is part of its tests).
 * It includes the oracle source so the whole oracle is instrumented, and
 * checks two exact identities along the way (iNTT(NTT(a)) = a; a rotation by
 * g followed by one by g^-1 with the same keys is not required to be exact,
 * so only shapes and ranges are checked there).  Exit status 0 = success.
 */
#include "ckks_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

/* SplitMix64 (Steele, Lea, Flood 2014): test input words only. */
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

/* n words per limb, limbs [count], residues below mods[i] */
static uint64_t *random_limbs(int count, uint64_t n, const uint64_t *mods, int lead)
{
    uint64_t *a = malloc(sizeof(uint64_t) * (uint64_t)lead * count * n);
    for (int r = 0; r < lead; r++)
        for (int i = 0; i < count; i++)
            for (uint64_t c = 0; c < n; c++) a[((uint64_t)r * count + i) * n + c] = next_u64() % mods[i];
    return a;
}

static int check_range(const uint64_t *a, int count, uint64_t n, const uint64_t *mods, int lead)
{
    for (int r = 0; r < lead; r++)
        for (int i = 0; i < count; i++)
            for (uint64_t c = 0; c < n; c++)
                if (a[((uint64_t)r * count + i) * n + c] >= mods[i]) return 0;
    return 1;
}

int main(void)
{
    const int log_n = 6, L = 6, K = 2, dnum = 3;
    const uint64_t n = (uint64_t)1 << log_n;
    uint64_t mod[8], psi[8];
    if (orc_gen_primes(log_n, 54, L, mod) != L || orc_gen_primes(log_n, 60, K, mod + L) != K) return 10;
    for (int i = 0; i < L + K; i++) psi[i] = orc_min_psi(mod[i], log_n);
    orc_params P = {log_n, L, K, dnum, mod, psi};
    const int level = L - 1, nq = L;
    const uint64_t ct = 2 * (uint64_t)nq * n;

    /* NTT round trip on all limbs */
    uint64_t *a = random_limbs(L + K, n, mod, 1);
    uint64_t *b = malloc(sizeof(uint64_t) * (L + K) * n);
    memcpy(b, a, sizeof(uint64_t) * (L + K) * n);
    orc_ntt_limbs(b, L + K, log_n, mod, psi, 0);
    orc_ntt_limbs(b, L + K, log_n, mod, psi, 1);
    if (memcmp(a, b, sizeof(uint64_t) * (L + K) * n) != 0) return 11;

    /* key switch, rotation (plain, accumulate, hoisted), rescale */
    uint64_t *evk = random_limbs(L + K, n, mod, 2 * dnum);
    uint64_t *evk2 = random_limbs(L + K, n, mod, 2 * dnum);
    uint64_t *x = random_limbs(nq, n, mod, 2);
    uint64_t *out = malloc(sizeof(uint64_t) * 4 * ct);
    orc_keyswitch(&P, level, x + nq * n, evk, out);
    if (!check_range(out, nq, n, mod, 2)) return 12;
    orc_rotate(&P, level, x, 5, evk, out, 0);
    orc_rotate(&P, level, x, 25, evk, out + ct, 1);
    if (!check_range(out, nq, n, mod, 4)) return 13;
    const uint32_t gs[2] = {5, 25};
    const uint64_t *ks[2] = {evk, evk2};
    orc_rotate_hoisted(&P, level, x, 2, gs, ks, out);
    if (!check_range(out, nq, n, mod, 4)) return 14;
    if (orc_rescale(&P, level, x, out) != 0 || !check_range(out, nq - 1, n, mod, 2)) return 15;

    /* multiply / relinearise / rescale on a batch of 2 */
    uint64_t *ya = random_limbs(nq, n, mod, 4), *yb = random_limbs(nq, n, mod, 4);
    if (orc_mul_relin_rescale(&P, level, ya, yb, evk, out, 2, 0) != 0) return 16;
    if (!check_range(out, nq - 1, n, mod, 4)) return 17;

    /* BSGS with plaintext and with encrypted diagonals: n_in 2, n_out 1, n1 2, n2 2 */
    uint64_t *pd = random_limbs(nq, n, mod, 2 * 2 * 2);
    uint64_t *cd = random_limbs(nq, n, mod, 2 * 2 * 2 * 2);
    uint64_t *xs = random_limbs(nq, n, mod, 4);
    const uint32_t gb[1] = {5}, gg[1] = {25};
    const uint64_t *kb[1] = {evk}, *kg[1] = {evk2};
    if (orc_ptmatvec(&P, level, xs, 2, pd, 1, 2, 2, gb, kb, gg, kg, out, 0, 0, 1) != 0) return 18;
    if (!check_range(out, nq - 1, n, mod, 2)) return 19;
    if (orc_ctmatvec(&P, level, xs, 2, cd, 1, 2, 2, evk, gb, kb, gg, kg, out, 0, 0, 1) != 0) return 20;
    if (!check_range(out, nq - 1, n, mod, 2)) return 21;

    /* polynomial evaluation, degree 3 on a batch of 2 */
    const double coeffs[4] = {0.5, -1.0, 0.25, 0.125};
    double out_scale = 0;
    if (orc_poly_eval(&P, level, ya, 2, 1125899906842624.0, coeffs, 3, evk, out, &out_scale) != 0) return 22;
    if (!check_range(out, nq - 3, n, mod, 4) || !(out_scale > 0)) return 23;

    free(a);
    free(b);
    free(evk);
    free(evk2);
    free(x);
    free(out);
    free(ya);
    free(yb);
    free(pd);
    free(cd);
    free(xs);
    printf("sanitized oracle run: ok\n");
    return 0;
}
