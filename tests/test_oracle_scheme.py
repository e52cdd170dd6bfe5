"""Pins for the oracle's key switching and the operations built on it.

Checks against what the mathematics fixes, never against the oracle itself:
  * with error-free keys, KS(d) decrypts to d*s' up to the ModDown rounding
    only: |k0 + k1*s - d*s'| <= (K/2)*(1 + h) per coefficient (also for
    hoisted rotations, where d = tau_g(c1) and s' = tau_g(s));
  * decrypt(rotate_k(ct)) = slots shifted left by k (C1 tolerance 2^-12,
    C3 parameters 2^-20), also for hoisted rotations, Rot_a(Rot_b) = Rot_(a+b),
    accumulate = ct + Rot;
  * mul/relinearise/rescale decrypts to the slot-wise product;
  * the BSGS matvec equals the float64 map y_o[s] = sum_c sum_t
    D_{o,c,t}[s] * x_c[(s+t) mod n], with plaintext and with encrypted
    diagonals; with trivially encrypted diagonals (c1 = 0) the encrypted-
    weight matvec gives the plaintext matvec's words exactly;
  * rotate-and-sum over all power-of-two offsets gives the slot sum in every slot;
  * Horner evaluation of p(x) = sum_k c_k x^k decrypts to p(z) slot-wise
    (float64 reference) at a scale equal to the primes' size;
  * the baby-step / giant-step evaluation (depth ceil(log2(d + 1))) decrypts
    to p(z) as well, and fits of exp on [-4, 0] and GELU on [-4, 4] decrypt to
    within their float64 approximation error of the functions; with primes
    that are exact in float64, p(x) = x + c returns the input's limbs
    (rescaling x*q_l by q_l is exact) plus the constant, and p(x) = c a
    trivial ciphertext; at degree 1 the tree and Horner agree word for word.
"""
import math
import numpy as np
import pytest

import ckks_synth as S
from helpers import (config_params, encrypt_slots, galois_key, params, rel_err, relin_key, secret)


def centered_max(orc, P, limbs_ntt, level):
    coeff = orc.ntt_params(P, limbs_ntt, inverse=True)
    x = orc.crt_centered(coeff, P.q[: level + 1])
    return max(abs(int(v)) for v in x)


@pytest.mark.parametrize("level", [23, 13, 4])
def test_keyswitch_noise_free_bound(orc, level):
    P = config_params(orc, "C3", log_n=9)
    h = 64
    s, s_ntt = secret(orc, P, 5, h)
    g = P.galois(3)
    evk = galois_key(orc, P, s_ntt, g, 5, "ks", zero_error=True)
    d = S.uniform_limbs(S.stream(level, "ks/d"), P.q[: level + 1], P.N)
    k = orc.keyswitch(P, level, d, evk)
    nq = level + 1
    mods = P.q[:nq]
    s_from = orc.automorph_ntt(s_ntt, P.log_n, g)[:nq]
    # e = k0 + k1*s - d*s'
    t1 = np.array([[int(a) * int(b) % m for a, b in zip(k[1, i], s_ntt[i])] for i, m in enumerate(mods)], dtype=np.uint64)
    t2 = np.array([[int(a) * int(b) % m for a, b in zip(d[i], s_from[i])] for i, m in enumerate(mods)], dtype=np.uint64)
    e = np.array([[(int(a) + int(b) - int(c)) % m for a, b, c in zip(k[0, i], t1[i], t2[i])]
                  for i, m in enumerate(mods)], dtype=np.uint64)
    assert centered_max(orc, P, e, level) <= (P.K / 2) * (1 + h)


@pytest.mark.parametrize("level", [5, 2])
def test_keyswitch_noise_free_bound_wide_primes(orc, level):
    """The same bound with primes at the top of the supported range (62-bit
    ciphertext and 61-bit special primes)."""
    P = orc.Params.generate(9, 6, 62, 2, 61, 3)
    h = 64
    s, s_ntt = secret(orc, P, 6, h)
    g = P.galois(5)
    evk = galois_key(orc, P, s_ntt, g, 6, "ksw", zero_error=True)
    d = S.uniform_limbs(S.stream(level, "ksw/d"), P.q[: level + 1], P.N)
    k = orc.keyswitch(P, level, d, evk)
    mods = P.q[: level + 1]
    s_from = orc.automorph_ntt(s_ntt, P.log_n, g)[: level + 1]
    t1 = np.array([[int(a) * int(b) % m for a, b in zip(k[1, i], s_ntt[i])] for i, m in enumerate(mods)], dtype=np.uint64)
    t2 = np.array([[int(a) * int(b) % m for a, b in zip(d[i], s_from[i])] for i, m in enumerate(mods)], dtype=np.uint64)
    e = np.array([[(int(a) + int(b) - int(c)) % m for a, b, c in zip(k[0, i], t1[i], t2[i])]
                  for i, m in enumerate(mods)], dtype=np.uint64)
    assert centered_max(orc, P, e, level) <= (P.K / 2) * (1 + h)


def test_hoisted_rotation_noise_free_bound(orc):
    """Hoisted rotations are key switches of tau_g(c1): with error-free keys
    k0 + k1*s = tau_g(c0) + tau_g(c1)*tau_g(s) up to the ModDown rounding."""
    P = config_params(orc, "C3", log_n=9)
    level, h = 17, 64
    s, s_ntt = secret(orc, P, 7, h)
    gs = [P.galois(k) for k in (1, 5, 100)]
    evks = [galois_key(orc, P, s_ntt, g, 7, "hk%d" % g, zero_error=True) for g in gs]
    ct = S.uniform_limbs(S.stream(7, "h/ct"), P.q[: level + 1], P.N, lead=(2,))
    out = orc.rotate_hoisted(P, level, ct, gs, evks)
    nq = level + 1
    mods = P.q[:nq]
    for r, g in enumerate(gs):
        c0g = orc.automorph_ntt(ct[0], P.log_n, g)
        c1g = orc.automorph_ntt(ct[1], P.log_n, g)
        sg = orc.automorph_ntt(s_ntt, P.log_n, g)[:nq]
        e = np.array([[(int(k0) + int(k1) * int(sv) - int(a0) - int(a1) * int(sgv)) % m
                       for k0, k1, sv, a0, a1, sgv in zip(out[r, 0, i], out[r, 1, i], s_ntt[i], c0g[i], c1g[i], sg[i])]
                      for i, m in enumerate(mods)], dtype=np.uint64)
        assert centered_max(orc, P, e, level) <= (P.K / 2) * (1 + h), g


def test_hoisted_rotations_decrypt_to_shifts(orc):
    P, s_ntt, z, ct, level, scale = c1_setup(orc, seed=3)
    ks = [1, 3, 7, P.N // 2 - 1]
    gs = [P.galois(k) for k in ks]
    evks = [galois_key(orc, P, s_ntt, g, 3, "hg%d" % g) for g in gs]
    out = orc.rotate_hoisted(P, level, ct, gs, evks)
    for r, k in enumerate(ks):
        assert rel_err(orc.decrypt(P, level, out[r], s_ntt, scale), np.roll(z, -k)) < 2 ** -12, k


def test_relin_key_noise_free_bound(orc):
    P = config_params(orc, "C3", log_n=9)
    level, h = 23, 64
    s, s_ntt = secret(orc, P, 6, h)
    rlk = relin_key(orc, P, s_ntt, 6, zero_error=True)
    d = S.uniform_limbs(S.stream(1, "rl/d"), P.q, P.N)
    k = orc.keyswitch(P, level, d, rlk)
    mods = P.q
    e = np.array([[(int(k0) + int(k1) * int(sv) - int(dv) * int(sv) * int(sv)) % m
                   for k0, k1, sv, dv in zip(k[0, i], k[1, i], s_ntt[i], d[i])]
                  for i, m in enumerate(mods)], dtype=np.uint64)
    assert centered_max(orc, P, e, level) <= (P.K / 2) * (1 + h)


def c1_setup(orc, seed=1):
    c = S.CONFIGS["C1"]
    P = config_params(orc, "C1")
    s, s_ntt = secret(orc, P, seed, c["h"])
    z = S.uniform_slots(S.stream(seed, "msg"), P.N // 2, complex_values=True)
    level = P.L - 1
    ct = encrypt_slots(orc, P, s_ntt, z, c["scale"], level, seed, "ct")
    return P, s_ntt, z, ct, level, c["scale"]


@pytest.mark.parametrize("k", [1, 7])
def test_c1_rotation_decrypts_to_shift(orc, k):
    P, s_ntt, z, ct, level, scale = c1_setup(orc)
    g = P.galois(k)
    evk = galois_key(orc, P, s_ntt, g, 1, "gk%d" % k)
    r = orc.rotate(P, level, ct, g, evk)
    assert rel_err(orc.decrypt(P, level, r, s_ntt, scale), np.roll(z, -k)) < 2 ** -12


def test_rotation_composition_and_accumulate(orc):
    P, s_ntt, z, ct, level, scale = c1_setup(orc, seed=2)
    g1, g6, g7 = P.galois(1), P.galois(6), P.galois(7)
    k1 = galois_key(orc, P, s_ntt, g1, 2, "k1")
    k6 = galois_key(orc, P, s_ntt, g6, 2, "k6")
    r = orc.rotate(P, level, orc.rotate(P, level, ct, g6, k6), g1, k1)
    assert rel_err(orc.decrypt(P, level, r, s_ntt, scale), np.roll(z, -7)) < 2 ** -11
    acc = orc.rotate(P, level, ct, g1, k1, flags=orc.ROT_ACCUMULATE)
    assert rel_err(orc.decrypt(P, level, acc, s_ntt, scale), z + np.roll(z, -1)) < 2 ** -11
    # g = 1 is the identity
    same = orc.rotate(P, level, ct, 1, k1)
    assert np.array_equal(same, ct)


@pytest.mark.slow
def test_c3_parameters_rotation(orc):
    c = S.CONFIGS["C3"]
    P = config_params(orc, "C3")
    s, s_ntt = secret(orc, P, 3, c["h"])
    z = S.uniform_slots(S.stream(3, "msg"), P.N // 2, complex_values=False)
    level = P.L - 1
    ct = encrypt_slots(orc, P, s_ntt, z, c["scale"], level, 3, "ct")
    k = 20001
    g = P.galois(k)
    evk = galois_key(orc, P, s_ntt, g, 3, "gk")
    r = orc.rotate(P, level, ct, g, evk)
    assert rel_err(orc.decrypt(P, level, r, s_ntt, c["scale"]), np.roll(z, -k)) < 2 ** -20


@pytest.mark.parametrize("log_n", [10, 12])
def test_mul_relin_rescale_decrypts_to_product(orc, log_n):
    c = S.CONFIGS["C5"]
    P = config_params(orc, "C5", log_n=log_n)
    s, s_ntt = secret(orc, P, 4, c["h"])
    level = P.L - 1
    n = P.N // 2
    za = S.uniform_slots(S.stream(4, "za"), n, complex_values=False)
    zb = S.uniform_slots(S.stream(4, "zb"), n, complex_values=False)
    scale = c["scale"]
    a = encrypt_slots(orc, P, s_ntt, za, scale, level, 4, "a")
    b = encrypt_slots(orc, P, s_ntt, zb, scale, level, 4, "b")
    rlk = relin_key(orc, P, s_ntt, 4)
    pre = orc.mul_relin_rescale(P, level, a[None], b[None], rlk, flags=orc.NO_RESCALE)[0]
    assert rel_err(orc.decrypt(P, level, pre, s_ntt, scale * scale), za * zb) < 2 ** -20
    post = orc.mul_relin_rescale(P, level, a[None], b[None], rlk)[0]
    assert post.shape == (2, level, P.N)
    assert np.array_equal(post, orc.rescale(P, level, pre))
    assert rel_err(orc.decrypt(P, level - 1, post, s_ntt, scale * scale / P.q[level]), za * zb) < 2 ** -12


def test_ptmatvec_matches_float_map(orc):
    P = config_params(orc, "C4", log_n=10)
    n = P.N // 2
    level, n_in, n_out, n1, n2 = 12, 2, 2, 4, 4
    s, s_ntt = secret(orc, P, 9, 64)
    scale = 2.0 ** 40
    rng = S.stream(9, "pmv/x")
    xs = [S.uniform_slots(rng, n, complex_values=False) for _ in range(n_in)]
    x = np.stack([encrypt_slots(orc, P, s_ntt, xs[c], scale, level, 9, "x%d" % c) for c in range(n_in)])
    D = S.normal_values(S.stream(9, "pmv/D"), (n_out, n_in, n1 * n2, n), 0.02)
    diags = np.empty((n_out, n_in, n2, n1, level + 1, P.N), dtype=np.uint64)
    for o in range(n_out):
        for c in range(n_in):
            for g in range(n2):
                for b in range(n1):
                    pre = np.roll(D[o, c, n1 * g + b], n1 * g)  # Rot_{-n1 g}
                    diags[o, c, g, b] = orc.encode(P, pre, scale, level)
    gb = [P.galois(b) for b in range(1, n1)]
    gg = [P.galois(n1 * g) for g in range(1, n2)]
    kb = [galois_key(orc, P, s_ntt, g, 9, "kb%d" % i) for i, g in enumerate(gb)]
    kg = [galois_key(orc, P, s_ntt, g, 9, "kg%d" % i) for i, g in enumerate(gg)]
    y_pre = orc.ptmatvec(P, level, x, diags, gb, kb, gg, kg, flags=orc.NO_RESCALE)
    y = orc.ptmatvec(P, level, x, diags, gb, kb, gg, kg)
    for o in range(n_out):
        ref = np.zeros(n)
        for c in range(n_in):
            for t in range(n1 * n2):
                ref += D[o, c, t] * np.roll(xs[c].real, -t)
        assert rel_err(orc.decrypt(P, level, y_pre[o], s_ntt, scale * scale).real, ref) < 2 ** -20
        assert np.array_equal(y[o], orc.rescale(P, level, y_pre[o]))
        assert rel_err(orc.decrypt(P, level - 1, y[o], s_ntt, scale * scale / P.q[level]).real, ref) < 2 ** -10
    # sampling a sub-range gives the same words
    y1 = orc.ptmatvec(P, level, x, diags, gb, kb, gg, kg, o_range=(1, 2))
    assert np.array_equal(y1[1], y[1])


def _bsgs_setup(orc, seed, level, n_in, n_out, n1, n2):
    P = config_params(orc, "C4", log_n=10)
    n = P.N // 2
    s, s_ntt = secret(orc, P, seed, 64)
    scale = 2.0 ** 40
    rng = S.stream(seed, "bsgs/x")
    xs = [S.uniform_slots(rng, n, complex_values=False) for _ in range(n_in)]
    x = np.stack([encrypt_slots(orc, P, s_ntt, xs[c], scale, level, seed, "x%d" % c) for c in range(n_in)])
    D = S.normal_values(S.stream(seed, "bsgs/D"), (n_out, n_in, n1 * n2, n), 0.02)
    gb = [P.galois(b) for b in range(1, n1)]
    gg = [P.galois(n1 * g) for g in range(1, n2)]
    kb = [galois_key(orc, P, s_ntt, g, seed, "kb%d" % i) for i, g in enumerate(gb)]
    kg = [galois_key(orc, P, s_ntt, g, seed, "kg%d" % i) for i, g in enumerate(gg)]
    return P, s_ntt, scale, xs, x, D, gb, gg, kb, kg


def _float_map(D, xs, o, n1, n2):
    ref = np.zeros(D.shape[-1])
    for c in range(len(xs)):
        for t in range(n1 * n2):
            ref += D[o, c, t] * np.roll(xs[c].real, -t)
    return ref


def test_ctmatvec_matches_float_map(orc):
    """Encrypted diagonals (each encrypted separately, pre-rotated by the
    inverse giant step): decrypts to the same float64 map as the plaintext
    matvec, at scale^2 before the rescale."""
    level, n_in, n_out, n1, n2 = 12, 2, 2, 4, 3
    P, s_ntt, scale, xs, x, D, gb, gg, kb, kg = _bsgs_setup(orc, 11, level, n_in, n_out, n1, n2)
    diags = np.empty((n_out, n_in, n2, n1, 2, level + 1, P.N), dtype=np.uint64)
    for o in range(n_out):
        for c in range(n_in):
            for g in range(n2):
                for b in range(n1):
                    pre = np.roll(D[o, c, n1 * g + b], n1 * g)  # Rot_{-n1 g}
                    diags[o, c, g, b] = encrypt_slots(orc, P, s_ntt, pre, scale, level, 11, "d%d.%d.%d.%d" % (o, c, g, b))
    rlk = relin_key(orc, P, s_ntt, 11)
    y_pre = orc.ctmatvec(P, level, x, diags, rlk, gb, kb, gg, kg, flags=orc.NO_RESCALE)
    y = orc.ctmatvec(P, level, x, diags, rlk, gb, kb, gg, kg)
    for o in range(n_out):
        ref = _float_map(D, xs, o, n1, n2)
        assert rel_err(orc.decrypt(P, level, y_pre[o], s_ntt, scale * scale).real, ref) < 2 ** -20
        assert np.array_equal(y[o], orc.rescale(P, level, y_pre[o]))
        assert rel_err(orc.decrypt(P, level - 1, y[o], s_ntt, scale * scale / P.q[level]).real, ref) < 2 ** -10
    y1 = orc.ctmatvec(P, level, x, diags, rlk, gb, kb, gg, kg, o_range=(1, 2))
    assert np.array_equal(y1[1], y[1])


def test_ctmatvec_trivial_diagonals_give_ptmatvec_words(orc):
    """A diagonal encrypted trivially, (pt, 0), makes every d2 zero, and the
    key switch of zero is zero: the result must be the plaintext matvec's
    words, bit for bit."""
    level, n_in, n_out, n1, n2 = 6, 2, 2, 3, 2
    P = config_params(orc, "C4", log_n=9)
    rng = S.stream(12, "bsgs/triv")
    x = S.uniform_limbs(rng, P.q[: level + 1], P.N, lead=(n_in, 2))
    pts = S.uniform_limbs(rng, P.q[: level + 1], P.N, lead=(n_out, n_in, n2, n1))
    ct_diags = np.zeros((n_out, n_in, n2, n1, 2, level + 1, P.N), dtype=np.uint64)
    ct_diags[:, :, :, :, 0] = pts
    gb = [P.galois(b) for b in range(1, n1)]
    gg = [P.galois(n1 * g) for g in range(1, n2)]
    kb = [S.uniform_limbs(S.stream(i, "bsgs/triv/kb"), P.mods, P.N, lead=(P.dnum, 2)) for i in range(n1 - 1)]
    kg = [S.uniform_limbs(S.stream(i, "bsgs/triv/kg"), P.mods, P.N, lead=(P.dnum, 2)) for i in range(n2 - 1)]
    rlk = S.uniform_limbs(S.stream(12, "bsgs/triv/rlk"), P.mods, P.N, lead=(P.dnum, 2))
    for flags in (0, orc.NO_RESCALE):
        a = orc.ctmatvec(P, level, x, ct_diags, rlk, gb, kb, gg, kg, flags=flags)
        b = orc.ptmatvec(P, level, x, pts, gb, kb, gg, kg, flags=flags)
        assert np.array_equal(a, b)
    # a nonzero c1 must change the words (the d2 path is live)
    ct_diags[0, 0, 0, 0, 1] = pts[0, 0, 0, 1]
    a = orc.ctmatvec(P, level, x, ct_diags, rlk, gb, kb, gg, kg)
    assert not np.array_equal(a[0], orc.ptmatvec(P, level, x, pts, gb, kb, gg, kg)[0])


def test_rotate_and_sum_gives_slot_sum(orc):
    P = config_params(orc, "C5", log_n=10)
    n = P.N // 2
    s, s_ntt = secret(orc, P, 8, 64)
    level, scale = 22, 2.0 ** 40
    z = S.uniform_slots(S.stream(8, "rs"), n, complex_values=False)
    ct = encrypt_slots(orc, P, s_ntt, z, scale, level, 8, "ct")
    steps = n.bit_length() - 1
    for k in range(steps):
        g = P.galois(1 << k)
        ct = orc.rotate(P, level, ct, g, galois_key(orc, P, s_ntt, g, 8, "r%d" % k), flags=orc.ROT_ACCUMULATE)
    dec = orc.decrypt(P, level, ct, s_ntt, scale).real
    assert np.max(np.abs(dec - z.sum())) / np.sum(np.abs(z)) < 2 ** -20


@pytest.mark.parametrize("coeffs", [
    [1.0, 1.0, 0.5, 1 / 6, 1 / 24, 1 / 120, 1 / 720, 1 / 5040],   # exp, degree 7 Taylor
    [0.25, -1.5],                                                  # affine
    [0.0, 0.5, 0.0, -0.125, 0.0, 0.03],                            # odd, degree 5
    [-1.75, 0.3, 1.9, -0.6],                                       # cubic, |c| up to 2
], ids=["exp7", "affine", "odd5", "cubic"])
def test_poly_eval_decrypts_to_polynomial(orc, coeffs):
    P = config_params(orc, "C3", log_n=9)
    level, h = 23, 64
    s, s_ntt = secret(orc, P, 9, h)
    rlk = relin_key(orc, P, s_ntt, 9)
    z = S.uniform_slots(S.stream(9, "pe/z"), P.N // 2, complex_values=False)
    scale = 2.0 ** 54
    ct = encrypt_slots(orc, P, s_ntt, z, scale, level, 9, "pe/ct")
    out, s_out = orc.poly_eval(P, level, ct[None], scale, coeffs, rlk)
    d = len(coeffs) - 1
    assert out.shape == (1, 2, level - d + 1, P.N)
    dec = orc.decrypt(P, level - d, out[0], s_ntt, s_out)
    ref = sum(c * z ** k for k, c in enumerate(coeffs))
    assert np.max(np.abs(dec - ref)) < 2 ** -30


def test_poly_eval_rejects_bad_input(orc):
    P = config_params(orc, "C1")
    s, s_ntt = secret(orc, P, 1, 64)
    rlk = relin_key(orc, P, s_ntt, 1)
    ct = S.uniform_limbs(S.stream(1, "pe/bad"), P.q, P.N, lead=(1, 2))
    with pytest.raises(ValueError):
        orc.poly_eval(P, 2, ct[:, :, :3], 2.0 ** 25, [1.0] * 5, rlk)  # degree 4 > level 2
    with pytest.raises(ValueError):
        orc.poly_eval(P, 3, ct, 2.0 ** 25, [0.0, 2.0 ** 40], rlk)     # c * q reaches 2^62


def _tree_setup(orc, seed):
    P = config_params(orc, "C3", log_n=9)
    s, s_ntt = secret(orc, P, seed, 64)
    return P, s_ntt, relin_key(orc, P, s_ntt, seed)


def _cheb_monomial(f, degree, lo, hi, drop=1e-12):
    """Monomial coefficients (in x) of f's Chebyshev interpolant on [lo, hi];
    coefficients below `drop` in magnitude set to zero."""
    from numpy.polynomial import chebyshev as C, polynomial as Pm
    p = C.Chebyshev.interpolate(f, degree, domain=[lo, hi]).convert(kind=Pm.Polynomial, domain=[-1, 1],
                                                                   window=[-1, 1])
    c = np.array(p.coef, dtype=np.float64)
    c[np.abs(c) < drop] = 0.0
    return [float(v) for v in c]


def _gelu(x):
    return 0.5 * x * (1.0 + np.vectorize(math.erf)(x / math.sqrt(2.0)))


@pytest.mark.parametrize("coeffs", [
    [1.0, 1.0, 0.5, 1 / 6, 1 / 24, 1 / 120, 1 / 720, 1 / 5040],   # exp, degree 7 Taylor
    [0.25, -1.5],                                                  # affine (depth 1)
    [0.0, 0.5, 0.0, -0.125, 0.0, 0.03],                            # odd, degree 5, zero terms skipped
    [-1.75, 0.3, 1.9, -0.6],                                       # cubic
    [0.1 * (-1) ** k / (k + 1) for k in range(17)],                # degree 16: the x^16 giant step
    [0.3, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, -0.7],                # x^8 alone: one-coefficient high part
    [0.2 * (k % 3 - 1) for k in range(32)],                        # degree 31, zero runs
], ids=["exp7", "affine", "odd5", "cubic", "deg16", "x8", "deg31"])
def test_poly_eval_tree_decrypts_to_polynomial(orc, coeffs):
    P, s_ntt, rlk = _tree_setup(orc, 10)
    level = 23
    z = S.uniform_slots(S.stream(10, "pt/z"), P.N // 2, complex_values=False)
    scale = 2.0 ** 54
    ct = encrypt_slots(orc, P, s_ntt, z, scale, level, 10, "pt/ct")
    out, s_out = orc.poly_eval_tree(P, level, ct[None], scale, coeffs, rlk)
    d = len(coeffs) - 1
    depth = int(np.ceil(np.log2(d + 1)))
    assert orc.tree_depth(d) == depth
    assert out.shape == (1, 2, level - depth + 1, P.N)
    assert s_out == scale
    dec = orc.decrypt(P, level - depth, out[0], s_ntt, s_out)
    ref = sum(c * z ** k for k, c in enumerate(coeffs))
    assert np.max(np.abs(dec - ref)) < 2 ** -30


def test_poly_eval_tree_exp_on_minus4_0(orc):
    """Degree-11 fit of exp on [-4, 0] (the input range of the softmax
    exponential): the decrypted output is within 2^-28 of the float64 fit and
    within 1e-8 of exp."""
    P, s_ntt, rlk = _tree_setup(orc, 11)
    level = 23
    coeffs = _cheb_monomial(np.exp, 11, -4.0, 0.0)
    rng = S.stream(11, "exp/z")
    x = -4.0 * rng.random(P.N // 2)
    x[:3] = [-4.0, 0.0, -2.0]
    scale = 2.0 ** 54
    ct = encrypt_slots(orc, P, s_ntt, x.astype(np.complex128), scale, level, 11, "exp/ct")
    out, s_out = orc.poly_eval_tree(P, level, ct[None], scale, coeffs, rlk)
    assert out.shape[2] == level - 4 + 1                          # degree 11: depth 4
    dec = orc.decrypt(P, level - 4, out[0], s_ntt, s_out).real
    fit = np.polynomial.polynomial.polyval(x, coeffs)
    assert np.max(np.abs(dec - fit)) < 2 ** -28
    assert np.max(np.abs(dec - np.exp(x))) < 1e-8


def test_poly_eval_tree_gelu_on_minus4_4(orc):
    """Degree-15 fit of GELU(4u) for u = x/4 in [-1, 1] (its odd terms above
    the first are zero and skipped): within 2^-30 of the float64 fit and
    within 3e-4 of GELU(x) = x Phi(x)."""
    P, s_ntt, rlk = _tree_setup(orc, 12)
    level = 23
    coeffs = _cheb_monomial(lambda u: _gelu(4.0 * u), 15, -1.0, 1.0)
    # GELU(x) - x/2 = x erf(x / sqrt 2) / 2 is even: the odd terms above the
    # first are conversion round-off
    for k in range(3, 16, 2):
        assert abs(coeffs[k]) < 1e-8
        coeffs[k] = 0.0
    rng = S.stream(12, "gelu/x")
    x = 8.0 * rng.random(P.N // 2) - 4.0
    x[:3] = [-4.0, 4.0, 0.0]
    u = x / 4.0
    scale = 2.0 ** 54
    ct = encrypt_slots(orc, P, s_ntt, u.astype(np.complex128), scale, level, 12, "gelu/ct")
    out, s_out = orc.poly_eval_tree(P, level, ct[None], scale, coeffs, rlk)
    assert out.shape[2] == level - 4 + 1                          # degree 15: depth 4
    dec = orc.decrypt(P, level - 4, out[0], s_ntt, s_out).real
    fit = np.polynomial.polynomial.polyval(u, coeffs)
    assert np.max(np.abs(dec - fit)) < 2 ** -30
    assert np.max(np.abs(dec - _gelu(x))) < 3e-4


def test_poly_eval_tree_exact_identities(orc):
    """C1 primes (30 bits) are exact in float64, so K_1 = round(1 * s * q_l / s)
    = q_l and rescaling x * q_l by q_l returns x's lower limbs word for word;
    p(x) = c alone is the trivial ciphertext (round(c s) mod q_i, 0)."""
    P = config_params(orc, "C1")
    s, s_ntt = secret(orc, P, 13, 64)
    rlk = relin_key(orc, P, s_ntt, 13)
    level = 3
    ct = S.uniform_limbs(S.stream(13, "id/ct"), P.q[: level + 1], P.N, lead=(2, 2))
    scale = 2.0 ** 25
    q = np.array(P.q[:level], dtype=np.uint64)[:, None]
    out, _ = orc.poly_eval_tree(P, level, ct, scale, [0.0, 1.0], rlk)
    assert np.array_equal(out, ct[:, :, :level])
    out, _ = orc.poly_eval_tree(P, level, ct, scale, [0.75, 1.0], rlk)
    k = np.uint64(round(0.75 * scale))
    assert np.array_equal(out[:, 0], (ct[:, 0, :level] + k % q) % q)
    assert np.array_equal(out[:, 1], ct[:, 1, :level])
    out, _ = orc.poly_eval_tree(P, level, ct, scale, [-0.5, 0.0], rlk)
    neg = np.uint64(round(0.5 * scale)) % q
    assert np.array_equal(out[:, 0], np.broadcast_to((q - neg) % q, out[:, 0].shape))
    assert not out[:, 1].any()


def test_poly_eval_tree_degree1_matches_horner(orc):
    P, s_ntt, rlk = _tree_setup(orc, 14)
    ct = S.uniform_limbs(S.stream(14, "d1/ct"), P.q[:6], P.N, lead=(2, 2))
    a, sa = orc.poly_eval(P, 5, ct, 2.0 ** 54, [0.3, -1.25], rlk)
    b, sb = orc.poly_eval_tree(P, 5, ct, 2.0 ** 54, [0.3, -1.25], rlk)
    assert np.array_equal(a, b) and sa == sb


def test_poly_eval_tree_rejects_bad_input(orc):
    P = config_params(orc, "C1")
    s, s_ntt = secret(orc, P, 1, 64)
    rlk = relin_key(orc, P, s_ntt, 1)
    ct = S.uniform_limbs(S.stream(1, "pt/bad"), P.q, P.N, lead=(1, 2))
    with pytest.raises(ValueError):
        orc.poly_eval_tree(P, 3, ct, 2.0 ** 25, [1.0] * 10, rlk)         # degree 9: depth 4 > level 3
    with pytest.raises(ValueError):
        orc.poly_eval_tree(P, 3, ct, 2.0 ** 25, [1.0] * 66, rlk)         # degree 65
    with pytest.raises(ValueError):
        orc.poly_eval_tree(P, 3, ct, 2.0 ** 25, [0.0, 2.0 ** 40], rlk)   # constant reaches 2^62
