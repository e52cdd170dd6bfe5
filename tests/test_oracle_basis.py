"""Pins for the oracle's basis conversions: ModUp, ModDown and rescale.

Readings (the pages give no formula): ModUp is the plain (unsigned) fast
basis conversion, ModDown converts the special-prime part with a centered
lift, rescale divides by the last prime with rounding to nearest.  Each is
checked against exact Python-integer identities on CRT values:
  ModUp   : out_t = X + u*Q' (mod m_t) for one u in [0, |I|), same for all t;
  ModDown : K = 1 gives exactly round(X / P); for any K,
            out*P = X - sum_k ybar_k*phat_k (mod Q_l) with
            ybar_k = centered([X * phat_k^-1]_{p_k}) and |sum| <= K*P/2;
  rescale : out = round(X / q_l) exactly.
"""
import numpy as np
import pytest

import ckks_synth as S


def prod(xs):
    r = 1
    for x in xs:
        r *= int(x)
    return r


def crt_unsigned(limbs, mods):
    M = prod(mods)
    acc = np.zeros(limbs.shape[-1], dtype=object)
    for x, m in zip(limbs, mods):
        Mi = M // m
        acc = acc + ((x.astype(object) * pow(Mi % m, -1, m)) % m) * Mi
    return acc % M


def small_c3(orc, log_n=8):
    c = S.CONFIGS["C3"]
    return orc.Params.generate(log_n, c["L"], c["q_bits"], c["K"], c["p_bits"], c["dnum"])


def wide_params(orc, log_n=8):
    """Primes at the top of the supported range: 6 x 62-bit ciphertext primes,
    2 x 61-bit special primes, dnum 3."""
    return orc.Params.generate(log_n, 6, 62, 2, 61, 3)


@pytest.mark.parametrize("level,wide", [(23, False), (12, False), (7, False), (20, False), (5, True), (2, True)])
def test_modup_is_plain_fast_basis_conversion(orc, level, wide):
    P = wide_params(orc) if wide else small_c3(orc)
    x = S.uniform_limbs(S.stream(level, "modup/x"), P.q[: level + 1], P.N)
    ext = P.ext_mods(level)
    for j in range(P.beta(level)):
        lo, hi = j * P.alpha, min((j + 1) * P.alpha, level + 1)
        out = orc.modup(P, level, j, x)
        assert out.shape == (level + 1 + P.K, P.N)
        Qd = prod(P.q[lo:hi])
        X = crt_unsigned(x[lo:hi], P.q[lo:hi])
        assert np.array_equal(out[lo:hi], x[lo:hi])
        # recover u from the first target limb outside the digit, then check all targets
        targets = [t for t in range(len(ext)) if not lo <= t < hi]
        for c in range(0, P.N, 7):
            Xc = int(X[c])
            m0 = ext[targets[0]]
            us = [u for u in range(hi - lo) if (Xc + u * Qd) % m0 == int(out[targets[0], c])]
            assert len(us) >= 1
            u = us[0]
            for t in targets:
                assert (Xc + u * Qd) % ext[t] == int(out[t, c])


def test_moddown_single_special_prime_is_exact_rounding(orc):
    P = orc.Params.generate(8, 4, 30, 1, 60, 4)
    level = 3
    ext = P.ext_mods(level)
    acc_coeff = S.uniform_limbs(S.stream(1, "md/acc"), ext, P.N)
    acc = orc.ntt(acc_coeff, ext, P.psi[: level + 1] + P.psi[P.L:], P.log_n)
    out = orc.moddown(P, level, acc)
    out_c = orc.ntt_params(P, out, inverse=True)
    X = crt_unsigned(acc_coeff, ext)
    M = prod(ext)
    Pp = P.p[0]
    got = orc.crt_centered(out_c, P.q[: level + 1])
    for c in range(P.N):
        Xc = int(X[c])
        if Xc > M // 2:
            Xc -= M
        # round to nearest (P odd: no ties)
        r = (2 * Xc + Pp) // (2 * Pp)
        assert int(got[c]) == r


@pytest.mark.parametrize("level,wide", [(23, False), (9, False), (5, True)])
def test_moddown_centered_identity(orc, level, wide):
    P = wide_params(orc) if wide else small_c3(orc)
    ext = P.ext_mods(level)
    psis = P.psi[: level + 1] + P.psi[P.L:]
    acc_coeff = S.uniform_limbs(S.stream(level, "md/acc8"), ext, P.N)
    acc = orc.ntt(acc_coeff, ext, psis, P.log_n)
    out = orc.moddown(P, level, acc)
    out_c = orc.ntt_params(P, out, inverse=True)
    Ql = prod(P.q[: level + 1])
    Pp = prod(P.p)
    X = crt_unsigned(acc_coeff, ext)
    O = crt_unsigned(out_c, P.q[: level + 1])
    for c in range(0, P.N, 3):
        Xc = int(X[c])
        eps = 0
        for pk in P.p:
            ph = Pp // pk
            y = (Xc % pk) * pow(ph % pk, -1, pk) % pk
            yb = y if y <= (pk - 1) // 2 else y - pk
            eps += yb * ph
        assert abs(eps) <= P.K * Pp // 2
        assert (int(O[c]) * Pp - (Xc - eps)) % Ql == 0


@pytest.mark.parametrize("level,wide", [(23, False), (1, False), (5, True)])
def test_rescale_is_exact_rounding(orc, level, wide):
    P = wide_params(orc) if wide else small_c3(orc)
    ct_coeff = S.uniform_limbs(S.stream(level, "rs/ct"), P.q[: level + 1], P.N, lead=(2,))
    ct = orc.ntt_params(P, ct_coeff)
    out = orc.rescale(P, level, ct)
    assert out.shape == (2, level, P.N)
    ql = P.q[level]
    for comp in range(2):
        X = orc.crt_centered(ct_coeff[comp], P.q[: level + 1])
        got = orc.crt_centered(orc.ntt_params(P, out[comp], inverse=True), P.q[:level])
        for c in range(P.N):
            assert int(got[c]) == (2 * int(X[c]) + ql) // (2 * ql)


def test_rescale_rejects_level_zero(orc):
    P = small_c3(orc)
    with pytest.raises(ValueError):
        orc.rescale(P, 0, np.zeros((2, 1, P.N), dtype=np.uint64))
