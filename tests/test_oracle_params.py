"""Pins for the oracle's parameter generation: the primes and the roots of unity.

The pages fix no parameter set; the readings are: ciphertext primes are the
largest primes below 2^bits that are 1 mod 2N (descending), special primes
the largest below 2^60, psi the smallest primitive 2N-th root.  These tests
prove each property with methods independent of the oracle's Miller-Rabin:
Lucas primality certificates from a full factorisation of m-1 (sympy),
Fermat witnesses for every skipped candidate, and an enumeration of all
primitive 2N-th roots from sympy's primitive root.
"""
import pytest
import sympy

import ckks_synth as S


def lucas_certificate(n):
    """True iff n is proven prime by Lucas' test with a full factorisation of n-1."""
    fs = sympy.factorint(n - 1)
    for a in range(2, 200):
        if pow(a, n - 1, n) != 1:
            return False
        if all(pow(a, (n - 1) // f, n) != 1 for f in fs):
            return True
    raise AssertionError("no Lucas witness found")


def composite_witness(c):
    return any(pow(b, c - 1, c) != 1 for b in (2, 3, 5, 7, 11, 13))


CASES = [(12, 30, 4), (12, 60, 1), (16, 54, 24), (16, 60, 8), (10, 54, 3), (12, 62, 3), (16, 61, 2)]


@pytest.mark.parametrize("log_n,bits,count", CASES)
def test_primes_are_prime_ntt_friendly_and_largest(orc, log_n, bits, count):
    ps = orc.gen_primes(log_n, bits, count)
    two_n = 2 << log_n
    assert ps == sorted(ps, reverse=True)
    for p in ps:
        assert p % two_n == 1 and p < 2 ** bits
        assert lucas_certificate(p)
    # every candidate = 1 mod 2N above the last prime and below 2^bits that was skipped is composite
    c = 2 ** bits - two_n + 1
    while c > ps[-1]:
        if c not in ps:
            assert composite_witness(c), c
        c -= two_n


def test_c1_values_match_independent_sympy_search(orc):
    # independent search with sympy.isprime
    def search(bits, log_n, count):
        out, c = [], 2 ** bits - (2 << log_n) + 1
        while len(out) < count:
            if sympy.isprime(c):
                out.append(c)
            c -= 2 << log_n
        return out

    assert orc.gen_primes(12, 30, 4) == search(30, 12, 4)
    assert orc.gen_primes(16, 54, 24) == search(54, 16, 24)


def test_is_prime_against_sympy(orc):
    import random

    rnd = random.Random(5)
    for _ in range(2000):
        n = rnd.getrandbits(rnd.choice([8, 20, 40, 62]))
        assert orc.is_prime(n) == sympy.isprime(n), n
    for n in [2, 3, 4, 561, 1105, 3215031751, 2152302898747, 3474749660383, 341550071728321]:
        assert orc.is_prime(n) == sympy.isprime(n), n


@pytest.mark.parametrize("log_n,bits,count", [(12, 30, 4), (12, 60, 1), (16, 54, 24), (16, 60, 8)])
def test_psi_is_smallest_primitive_2n_th_root(orc, log_n, bits, count):
    n = 1 << log_n
    for m in orc.gen_primes(log_n, bits, count):
        psi = orc.min_psi(m, log_n)
        assert pow(psi, n, m) == m - 1 and pow(psi, 2 * n, m) == 1
        g = sympy.primitive_root(m)
        w = pow(g, (m - 1) // (2 * n), m)  # primitive 2N-th root
        w2, cur, best = w * w % m, w, m
        for _ in range(n):  # all odd powers of w
            best = min(best, cur)
            cur = cur * w2 % m
        assert psi == best


# Literal parameter values of the workload recipes, computed independently of
# the oracle (sympy's primality test over the candidates 1 mod 2N below 2^bits,
# and the minimum over all odd powers of a primitive 2N-th root from sympy's
# primitive root): any change to the prime search or the root choice fails here.
C1_Q = [1073692673, 1073668097, 1073651713, 1073643521]
C1_P = [1152921504606830593]
C3_Q = [18014398506729473, 18014398505943041, 18014398496243713, 18014398495457281, 18014398492704769,
        18014398492311553, 18014398491918337, 18014398487068673, 18014398485495809, 18014398484316161,
        18014398479204353, 18014398476451841, 18014398472519681, 18014398471864321, 18014398470946817,
        18014398467407873, 18014398463868929, 18014398462427137, 18014398458888193, 18014398457184257,
        18014398452203521, 18014398450892801, 18014398446305281, 18014398445387777]
C3_P = [1152921504606584833, 1152921504598720513, 1152921504597016577, 1152921504595968001, 1152921504592822273,
        1152921504592429057, 1152921504589938689, 1152921504586530817]


def test_c1_literal_primes_and_psi(orc):
    c = S.CONFIGS["C1"]
    P = orc.Params.generate(c["log_n"], c["L"], c["q_bits"], c["K"], c["p_bits"], c["dnum"])
    assert P.q == C1_Q and P.p == C1_P
    assert P.psi[0] == 236231 and P.psi[P.L] == 116777451583545
    assert P.galois(1) == 5 and P.galois(7) == 4397


def test_c3_appendix_psi_values(orc):
    c = S.CONFIGS["C3"]
    P = orc.Params.generate(c["log_n"], c["L"], c["q_bits"], c["K"], c["p_bits"], c["dnum"])
    assert P.q == C3_Q and P.p == C3_P
    assert P.psi[0] == 197149534992 and P.psi[P.L] == 18043022392882
    assert P.alpha == 8 and P.beta(23) == 3 and P.beta(12) == 2 and P.beta(7) == 1
    for m in C3_Q[:2] + C3_P[:1]:  # the literal values themselves, independently of the oracle
        assert sympy.isprime(m) and m % (1 << 17) == 1
