"""Parity where the lazy (partially reduced) arithmetic of the kernels comes
closest to overflowing 64 bits, through the C interface, word for word
against the oracle.

The kernels keep intermediate words above the modulus: lazy forward
butterflies let words grow by up to 4q per stage for q < 2^57 (about 70q at
the end of a transform), lazy inverse butterflies let the bound double per
stage for q < 2^54, basis-conversion outputs stay below 6q and the key inner
product sums Montgomery products below 2m.  Uniform residues rarely reach
those bounds; here every input word lies in the top 2^16 residues of its
modulus, some limbs are all m-1, and the parameter sets put ciphertext
primes just below 2^55, 2^56 and 2^57 (forward butterflies lazy at the
tightest bound, inverse butterflies strict) next to the 54-bit sets of the
workloads.  The wide sets put primes at 2^59-2^62: Harvey butterflies up to
2^61, exact-quotient butterflies and a Montgomery reduction after every digit
above, full-width dot products once any prime reaches 2^60.
"""
import numpy as np
import pytest

import ckks_synth as S
from gpu_util import announce, config_pair, empty_dev, make_pair, to_dev, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch_cuda()
    import private_rns_ckks_amd as L

    return L


@pytest.fixture(scope="module")
def c3small(lib, orc):
    return config_pair(lib, orc, "C3", log_n=12)


def top(P, moduli, seed, tag, lead=()):
    """Top-of-range words; limb 0 of the first item is all m-1."""
    x = S.top_limbs(S.stream(seed, tag), moduli, P.N, lead=lead)
    first = x.reshape((-1,) + x.shape[-2:])[0]
    first[0, :] = np.uint64(moduli[0] - 1)
    return x


# (log_n, L, q_bits, K, p_bits, dnum): the 54-bit workload primes at N=2^12 and
# 2^16, and ciphertext primes just below 2^55, 2^56 and 2^57
TOP_SETS = [
    (12, 24, 54, 8, 60, 3),
    (13, 12, 55, 4, 60, 3),
    (12, 12, 56, 6, 60, 2),
    (14, 12, 57, 4, 60, 3),
]
# primes at the top of the supported range (below 2^62)
WIDE_SETS = [
    (12, 6, 62, 2, 61, 3),
    (13, 8, 61, 4, 62, 2),
    (12, 8, 60, 4, 59, 2),
]
ALL_SETS = TOP_SETS + WIDE_SETS


@pytest.mark.parametrize("ps", ALL_SETS, ids=lambda s: "logn%d_q%d_p%d" % (s[0], s[2], s[4]))
def test_ntt_top_of_range(lib, orc, ps):
    ctx, P = make_pair(lib, orc, *ps)
    announce("ntt top-of-range %s" % (ps,))
    nl = P.L + P.K
    x = top(P, P.mods, 1, "gpu/top/ntt", lead=(2,))
    d = to_dev(x)
    lib.ckks_ntt(ctx, d, 2, 0, nl, 0)
    assert np.array_equal(to_host(d), orc.ntt_params(P, x))
    d2 = to_dev(x)
    lib.ckks_ntt(ctx, d2, 2, 0, nl, 1)
    assert np.array_equal(to_host(d2), orc.ntt_params(P, x, inverse=True))
    ctx.close()


def test_ntt_top_of_range_n16(lib, orc):
    """The N = 2^16 specialisation of the passes, top-of-range words on the 24 workload primes."""
    ctx, P = config_pair(lib, orc, "C2")
    announce("ntt top-of-range N=2^16")
    x = top(P, P.q, 2, "gpu/top/ntt16", lead=(2,))
    for inverse in (0, 1):
        d = to_dev(x)
        lib.ckks_ntt(ctx, d, 2, 0, P.L, inverse)
        assert np.array_equal(to_host(d), orc.ntt_params(P, x, inverse=bool(inverse))), inverse
    ctx.close()


@pytest.mark.parametrize("ps", ALL_SETS, ids=lambda s: "logn%d_q%d_p%d" % (s[0], s[2], s[4]))
def test_keyswitch_top_of_range(lib, orc, ps):
    ctx, P = make_pair(lib, orc, *ps)
    for level in (P.L - 1, P.L // 2):
        announce("keyswitch top-of-range %s level=%d" % (ps, level))
        d = top(P, P.q[: level + 1], level, "gpu/top/ks/d")
        evk = top(P, P.mods, level, "gpu/top/ks/k", lead=(P.dnum, 2))
        out = empty_dev((2, level + 1, P.N))
        lib.ckks_keyswitch(ctx, to_dev(d), to_dev(evk), out, level)
        assert np.array_equal(to_host(out), orc.keyswitch(P, level, d, evk)), level
    ctx.close()


@pytest.mark.parametrize("flags", [0, 1])
@pytest.mark.parametrize("ps", ALL_SETS, ids=lambda s: "logn%d_q%d_p%d" % (s[0], s[2], s[4]))
def test_rotate_top_of_range(lib, orc, ps, flags):
    ctx, P = make_pair(lib, orc, *ps)
    level = P.L - 1
    announce("rotate top-of-range %s flags=%d" % (ps, flags))
    ks = [1, 5, P.N // 2 - 1]
    B = len(ks)
    cts = top(P, P.q[: level + 1], 3, "gpu/top/rot/ct", lead=(B, 2))
    gs = [P.galois(k) for k in ks]
    keys = [top(P, P.mods, b, "gpu/top/rot/k", lead=(P.dnum, 2)) for b in range(B)]
    out = empty_dev(cts.shape)
    lib.ckks_rotate(ctx, to_dev(cts), out, B, level, gs, [to_dev(k) for k in keys], flags)
    ref = orc.rotate_batch(P, level, cts, gs, keys, orc.ROT_ACCUMULATE if flags else 0)
    assert np.array_equal(to_host(out), ref)
    ctx.close()


@pytest.mark.parametrize("ps", TOP_SETS[:2] + WIDE_SETS, ids=lambda s: "logn%d_q%d_p%d" % (s[0], s[2], s[4]))
def test_rescale_and_mul_top_of_range(lib, orc, ps):
    ctx, P = make_pair(lib, orc, *ps)
    level = P.L - 1
    announce("rescale / mul_relin_rescale top-of-range %s" % (ps,))
    B = 2
    a = top(P, P.q, 4, "gpu/top/mrr/a", lead=(B, 2))
    b = top(P, P.q, 4, "gpu/top/mrr/b", lead=(B, 2))
    rlk = top(P, P.mods, 4, "gpu/top/mrr/k", lead=(P.dnum, 2))
    out = empty_dev((B, 2, level, P.N))
    lib.ckks_rescale(ctx, to_dev(a), out, B, level)
    got = to_host(out)
    for i in range(B):
        assert np.array_equal(got[i], orc.rescale(P, level, a[i])), i
    for flags in (0, 2):
        lo = level + 1 if flags else level
        out = empty_dev((B, 2, lo, P.N))
        lib.ckks_mul_relin_rescale(ctx, to_dev(a), to_dev(b), to_dev(rlk), out, B, level, flags)
        assert np.array_equal(to_host(out), orc.mul_relin_rescale(P, level, a, b, rlk, flags)), flags
    ctx.close()


def test_keyswitch_top_of_range_c3_full(lib, orc):
    """One top-of-range key switch and one accumulating rotation at the full
    workload shape (N = 2^16, L = 24, K = 8, level 23), in the benchmark's
    launch configuration."""
    ctx, P = config_pair(lib, orc, "C3")
    level = P.L - 1
    announce("keyswitch + rotate top-of-range at N=2^16")
    d = top(P, P.q, 5, "gpu/top/full/d")
    evk = top(P, P.mods, 5, "gpu/top/full/k", lead=(P.dnum, 2))
    out = empty_dev((2, level + 1, P.N))
    lib.ckks_keyswitch(ctx, to_dev(d), to_dev(evk), out, level)
    assert np.array_equal(to_host(out), orc.keyswitch(P, level, d, evk))
    ct = top(P, P.q, 6, "gpu/top/full/ct", lead=(1, 2))
    g = P.galois(12345)
    out = empty_dev(ct.shape)
    lib.ckks_rotate(ctx, to_dev(ct), out, 1, level, [g], [to_dev(evk)], lib.CKKS_ROT_ACCUMULATE)
    ref = orc.rotate_batch(P, level, ct, [g], [evk], orc.ROT_ACCUMULATE)
    assert np.array_equal(to_host(out), ref)
    ctx.close()


@pytest.mark.parametrize("ps", WIDE_SETS, ids=lambda s: "logn%d_q%d_p%d" % (s[0], s[2], s[4]))
def test_wide_primes_composite_ops(lib, orc, ps):
    """The operations built on the key switch, with primes at 2^59-2^62 and
    top-of-range words: hoisted rotations, both BSGS products and the
    depth-efficient polynomial evaluation, word for word against the oracle."""
    ctx, P = make_pair(lib, orc, *ps)
    level = P.L - 1
    announce("wide-prime composite ops %s" % (ps,))
    # hoisted rotations of 2 inputs by 3 elements (one the identity)
    gs = [P.galois(k) for k in (1, 0, 7)]
    cts = top(P, P.q, 7, "gpu/wide/hoist/ct", lead=(2, 2))
    keys = [top(P, P.mods, r, "gpu/wide/hoist/k", lead=(P.dnum, 2)) for r in range(len(gs))]
    out = empty_dev((2, len(gs)) + cts.shape[1:])
    lib.ckks_rotate_hoisted(ctx, to_dev(cts), 2, level, gs, [to_dev(k) for k in keys], out)
    got = to_host(out)
    for c in range(2):
        assert np.array_equal(got[c], orc.rotate_hoisted(P, level, cts[c], gs, keys)), c
    # BSGS products: 2 inputs, 2 outputs, 3 x 2 steps
    n_in, n_out, n1, n2 = 2, 2, 3, 2
    x = top(P, P.q, 8, "gpu/wide/mv/x", lead=(n_in, 2))
    gb = [P.galois(b) for b in range(1, n1)]
    gg = [P.galois(n1 * g) for g in range(1, n2)]
    kb = [top(P, P.mods, i, "gpu/wide/mv/kb", lead=(P.dnum, 2)) for i in range(n1 - 1)]
    kg = [top(P, P.mods, i, "gpu/wide/mv/kg", lead=(P.dnum, 2)) for i in range(n2 - 1)]
    pd = top(P, P.q, 9, "gpu/wide/mv/pd", lead=(n_out, n_in, n2, n1))
    y = empty_dev((n_out, 2, level, P.N))
    lib.ckks_ptmatvec(ctx, to_dev(x), n_in, to_dev(pd), n_out, n1, n2, gb, [to_dev(k) for k in kb], gg,
                      [to_dev(k) for k in kg], y, level)
    assert np.array_equal(to_host(y), orc.ptmatvec(P, level, x, pd, gb, kb, gg, kg))
    cd = top(P, P.q, 10, "gpu/wide/mv/cd", lead=(n_out, n_in, n2, n1, 2))
    rlk = top(P, P.mods, 11, "gpu/wide/mv/rlk", lead=(P.dnum, 2))
    y = empty_dev((n_out, 2, level, P.N))
    lib.ckks_ctmatvec(ctx, to_dev(x), n_in, to_dev(cd), n_out, n1, n2, to_dev(rlk), gb, [to_dev(k) for k in kb], gg,
                      [to_dev(k) for k in kg], y, level)
    assert np.array_equal(to_host(y), orc.ctmatvec(P, level, x, cd, rlk, gb, kb, gg, kg))
    # polynomial of degree 5 (depth 3) at scale 2^(bits of q_0 - 1); the
    # coefficients are small enough that every rounded constant stays below 2^62
    coeffs = [c / 8 for c in (0.5, -1.0, 0.25, 0.125, -0.5, 0.0625)]
    scale = float(2 ** (P.q[0].bit_length() - 1))
    depth = lib.tree_depth(len(coeffs) - 1)
    out = empty_dev((2, 2, level - depth + 1, P.N))
    lib.ckks_poly_eval_tree(ctx, to_dev(cts), 2, level, scale, coeffs, to_dev(rlk), out)
    ref, _ = orc.poly_eval_tree(P, level, cts, scale, coeffs, rlk)
    assert np.array_equal(to_host(out), ref)
    ctx.close()
