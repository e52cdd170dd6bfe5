"""Pins for the oracle's Galois automorphism, CRT and canonical-embedding
encode/decode.

Readings (the pages give no formula): tau_g maps a(X) to a(X^g) mod X^N+1;
slot j lives at zeta^(5^j mod 2N) with zeta = exp(i*pi/N); rotation by k is
g = 5^k mod 2N and moves slot j+k to slot j.  Checks: evaluation of a(X^g)
at roots of X^N+1 by Horner (independent of the permutation formula), the
NTT-form permutation against NTT(tau(iNTT(x))), group composition, the
direct O(N^2) embedding matrix, exact recovery of known signed integers by
the CRT, and decode(tau_{5^k}(encode(z))) = z shifted by k.
"""
import numpy as np
import pytest

import ckks_synth as S


def horner(coeffs, x, m):
    acc = 0
    for c in reversed(coeffs):
        acc = (acc * x + int(c)) % m
    return acc


@pytest.mark.parametrize("log_n,g", [(3, 3), (4, 5), (6, 25), (8, 5 ** 7 % 512), (8, 511), (10, 3)])
def test_coeff_automorphism_evaluates_as_substitution(orc, log_n, g):
    n = 1 << log_n
    m = orc.gen_primes(16, 54, 1)[0]
    psi = orc.min_psi(m, log_n)
    a = S.uniform_limbs(S.stream(log_n, "aut/sub"), [m], n)
    b = orc.automorph_coeff(a, [m], log_n, g)[0]
    for e in (1, 3, 2 * n - 1, 5, 7):
        r = pow(psi, e, m)  # a root of X^N + 1
        assert horner(b, r, m) == horner(a[0], pow(r, g, m), m)


@pytest.mark.parametrize("log_n", [4, 12])
def test_ntt_form_automorphism_is_conjugated_coefficient_automorphism(orc, log_n):
    P = orc.Params.generate(log_n, 3, 54, 1, 60, 1)
    x = S.uniform_limbs(S.stream(log_n, "aut/ntt"), P.mods, P.N)
    for g in (5, 25, 2 * P.N - 1, pow(5, 1234, 2 * P.N) if log_n > 10 else 3):
        via = orc.ntt_params(P, orc.automorph_coeff(orc.ntt_params(P, x, inverse=True), P.mods, log_n, g))
        assert np.array_equal(orc.automorph_ntt(x, log_n, g), via)


def test_automorphism_composition(orc):
    log_n = 10
    m = orc.gen_primes(16, 54, 1)[0]
    a = S.uniform_limbs(S.stream(2, "aut/comp"), [m], 1 << log_n)
    two_n = 2 << log_n
    g, h = 5, 5 ** 9 % two_n
    lhs = orc.automorph_coeff(orc.automorph_coeff(a, [m], log_n, h), [m], log_n, g)
    rhs = orc.automorph_coeff(a, [m], log_n, g * h % two_n)
    assert np.array_equal(lhs, rhs)
    assert np.array_equal(orc.automorph_coeff(a, [m], log_n, 1), a)


def test_crt_recovers_known_signed_integers(orc):
    P = orc.Params.generate(12, 4, 30, 1, 60, 4)
    rnd = np.random.default_rng(1)
    Q = 1
    for q in P.q:
        Q *= q
    vals = [int(v) for v in rnd.integers(-2 ** 62, 2 ** 62, size=64)]
    vals += [(Q - 1) // 2, -((Q - 1) // 2), 0, 1, -1, 2 ** 100 + 12345, -(2 ** 110)]
    limbs = np.array([[v % q for v in vals] for q in P.q], dtype=np.uint64)
    got = orc.crt_centered(limbs, P.q)
    assert [int(v) for v in got] == vals


def direct_decode(m, N, scale):
    e = orc_slot_exponents(N)
    k = np.arange(N)
    M = np.exp(1j * np.pi * np.outer(e, k) / N)
    return M @ np.asarray(m, dtype=np.float64) / scale


def orc_slot_exponents(N):
    return np.array([pow(5, j, 2 * N) for j in range(N // 2)])


@pytest.mark.parametrize("log_n", [4, 10])
def test_decode_matches_direct_embedding(orc, log_n):
    N = 1 << log_n
    m = S.rounded_gaussian(S.stream(log_n, "enc/m"), N, 1000.0)
    got = orc.decode_coeffs(m, N, 1.0)
    ref = direct_decode(m, N, 1.0)
    assert np.allclose(got, ref, rtol=0, atol=1e-8 * np.max(np.abs(ref)))


@pytest.mark.parametrize("log_n", [4, 10])
def test_encode_matches_direct_inverse_embedding(orc, log_n):
    N = 1 << log_n
    n = N // 2
    scale = 2.0 ** 20
    z = S.uniform_slots(S.stream(log_n, "enc/z"), n)
    e = orc_slot_exponents(N)
    k = np.arange(N)
    raw = (2.0 / N) * np.real(np.exp(-1j * np.pi * np.outer(k, e) / N) @ (scale * z))
    got = orc.encode_coeffs(z, N, scale)
    frac = np.abs(raw - np.floor(raw) - 0.5)
    ok = frac > 1e-6  # away from rounding ties
    assert np.array_equal(got[ok], np.rint(raw[ok]).astype(np.int64))
    # and decode inverts encode up to the rounding of N coefficients
    back = orc.decode_coeffs(got, N, scale)
    assert np.max(np.abs(back - z)) <= N / (2 * scale)


@pytest.mark.parametrize("k", [1, 7, 100, -3])
def test_rotation_galois_element_shifts_slots(orc, k):
    P = orc.Params.generate(10, 2, 54, 0, 60, 1)
    z = S.uniform_slots(S.stream(11, "enc/rot"), P.N // 2)
    scale = 2.0 ** 30
    pt = orc.encode(P, z, scale, 1)
    g = P.galois(k)
    assert g == pow(5, k % (P.N // 2), 2 * P.N)
    rot = orc.automorph_ntt(pt, P.log_n, g)
    coeff = orc.ntt_params(P, rot, inverse=True)
    dec = orc.decode_limbs(P, coeff, scale, 1)
    assert np.max(np.abs(dec - np.roll(z, -k))) < 1e-6
