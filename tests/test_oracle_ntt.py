"""Pins for the oracle's negacyclic NTT.

Definition pinned (reading of the pages, which give no transform): word j of
the forward transform is the polynomial evaluated at psi^(2*brv(j)+1); the
inverse returns natural-order coefficients including the factor 1/N.
Checks: direct O(N^2) evaluation of that definition in Python integers,
schoolbook negacyclic convolution, round trips at the configured sizes, the
closed form for NTT(X), and Horner evaluation at sampled indices at N=2^16.
"""
import random

import numpy as np
import pytest

import ckks_synth as S


def brv(x, bits):
    return int(format(x, "0%db" % bits)[::-1], 2) if bits else 0


def direct_ntt(a, m, psi, log_n):
    n = 1 << log_n
    out = []
    for j in range(n):
        r = pow(psi, 2 * brv(j, log_n) + 1, m)
        acc, x = 0, 1
        for i in range(n):
            acc = (acc + int(a[i]) * x) % m
            x = x * r % m
        out.append(acc)
    return out


def negacyclic(a, b, m):
    n = len(a)
    c = [0] * n
    for i in range(n):
        for j in range(n):
            v = int(a[i]) * int(b[j])
            if i + j < n:
                c[i + j] += v
            else:
                c[i + j - n] -= v
    return [x % m for x in c]


@pytest.mark.parametrize("log_n", [1, 2, 3, 5, 7, 9])
@pytest.mark.parametrize("bits", [30, 54, 60, 61, 62])
def test_forward_matches_direct_evaluation(orc, log_n, bits):
    m = orc.gen_primes(16, bits, 1)[0]  # 1 mod 2^17, hence 1 mod 2N for every N here
    psi = orc.min_psi(m, log_n)
    rng = S.stream(log_n * 100 + bits, "ntt/direct")
    a = S.uniform_limbs(rng, [m], 1 << log_n)
    got = orc.ntt(a, [m], [psi], log_n)[0]
    assert [int(v) for v in got] == direct_ntt(a[0], m, psi, log_n)
    back = orc.ntt(got[None, :], [m], [psi], log_n, inverse=True)[0]
    assert np.array_equal(back, a[0])


@pytest.mark.parametrize("log_n", [3, 6, 8])
def test_product_is_negacyclic_convolution(orc, log_n):
    m = orc.gen_primes(16, 54, 2)[1]
    psi = orc.min_psi(m, log_n)
    rng = S.stream(log_n, "ntt/conv")
    a, b = S.uniform_limbs(rng, [m, m], 1 << log_n)
    fa = orc.ntt(a[None], [m], [psi], log_n)[0]
    fb = orc.ntt(b[None], [m], [psi], log_n)[0]
    prod = np.array([int(x) * int(y) % m for x, y in zip(fa, fb)], dtype=np.uint64)
    c = orc.ntt(prod[None], [m], [psi], log_n, inverse=True)[0]
    assert [int(v) for v in c] == negacyclic(a, b, m)


@pytest.mark.parametrize("name", ["C1", "C3"])
def test_round_trip_at_config_sizes(orc, name):
    c = S.CONFIGS[name]
    P = orc.Params.generate(c["log_n"], c["L"], c["q_bits"], c["K"], c["p_bits"], c["dnum"])
    a = S.uniform_limbs(S.stream(1, "ntt/rt"), P.mods, P.N)
    f = orc.ntt_params(P, a)
    assert not np.array_equal(f, a)
    assert all((f[t] < m).all() for t, m in enumerate(P.mods))
    assert np.array_equal(orc.ntt_params(P, f, inverse=True), a)


def test_transform_of_x_is_the_roots(orc):
    log_n = 16
    P = orc.Params.generate(log_n, 2, 54, 1, 60, 1)
    n = P.N
    x = np.zeros((3, n), dtype=np.uint64)
    x[:, 1] = 1
    f = orc.ntt_params(P, x)
    idx = np.arange(n)
    br = np.array([brv(j, log_n) for j in range(0, n, 97)])
    for t, m in enumerate(P.mods):
        for j, b in zip(range(0, n, 97), br):
            assert int(f[t, j]) == pow(P.psi[t], 2 * int(b) + 1, m)
    assert idx.size == n


def test_sampled_horner_at_2_16(orc):
    log_n = 16
    P = orc.Params.generate(log_n, 1, 54, 1, 60, 1)
    n = P.N
    a = S.uniform_limbs(S.stream(7, "ntt/horner"), P.mods, n)
    f = orc.ntt_params(P, a)
    rnd = random.Random(3)
    coeffs = [[int(v) for v in a[t]] for t in range(2)]
    for t, m in enumerate(P.mods):
        for j in rnd.sample(range(n), 6):
            r = pow(P.psi[t], 2 * brv(j, log_n) + 1, m)
            acc = 0
            for c in reversed(coeffs[t]):
                acc = (acc * r + c) % m
            assert int(f[t, j]) == acc
