"""Parity at the full workload sizes, in the launch configuration the
benchmark uses, on sampled outputs the oracle computes one by one.

C3: the 32-ciphertext rotation batch (N=2^16, L=24, K=8, dnum=3), every item
    checked, item 0 a real encryption under a real Galois key (decrypt =
    shifted slots).
C5: 48 ciphertext pairs: multiply + relinearise + rescale, then rotate-and-sum
    over the 15 power-of-two offsets, pairs 0, 24 and 47 checked, pair 0 real
    (decrypt = slot sum).
C4: the BSGS matvec at level 12 with 12 x 3 x 8 x 8 diagonals (15.7 GB),
    outputs 0 and 11 checked.
Polynomial evaluation: degree 7 on the 48 ciphertexts of a C5 batch at level
    23 (scale 2^54), with item 0 a real encryption (decrypts to p(slots)).
A x V: the encrypted-weight BSGS matvec at level 12 with 3 x 3 x 8 x 8
    ciphertext diagonals (7.9 GB), outputs 0 and 2 checked.
"""
import numpy as np
import pytest

import ckks_synth as S
from gpu_util import announce, config_pair, empty_dev, to_dev, to_host, torch_cuda
from helpers import encrypt_slots, galois_key, rel_err, relin_key, secret

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch_cuda()
    import private_rns_ckks_amd as L

    return L


@pytest.fixture(scope="module")
def full(lib, orc):
    return config_pair(lib, orc, "C3")


def test_c3_full_batch(lib, orc, full):
    ctx, P = full
    c = S.CONFIGS["C3"]
    B, level = c["batch"], P.L - 1
    announce("C3 full batch: %d rotations at N=2^16" % B)
    s, s_ntt = secret(orc, P, 3, c["h"])
    offsets = S.distinct_offsets(S.stream(3, "full/offsets"), B, *c["offset_range"])
    gs = [P.galois(int(k)) for k in offsets]
    cts = S.uniform_limbs(S.stream(3, "full/ct"), P.q, P.N, lead=(B, 2))
    z = S.uniform_slots(S.stream(3, "full/msg"), P.N // 2, complex_values=False)
    cts[0] = encrypt_slots(orc, P, s_ntt, z, c["scale"], level, 3, "full/enc")
    keys_h = [galois_key(orc, P, s_ntt, gs[0], 3, "full/gk0")]
    keys_h += [S.uniform_limbs(S.stream(b, "full/evk"), P.mods, P.N, lead=(P.dnum, 2)) for b in range(1, B)]
    d_out = empty_dev(cts.shape)
    lib.ckks_rotate(ctx, to_dev(cts), d_out, B, level, gs, [to_dev(k) for k in keys_h])
    got = to_host(d_out)
    for t, m in enumerate(P.q):
        assert (got[:, :, t, :] < m).all()
    # every item of the batch, word for word (each has its own offset and key)
    ref = orc.rotate_batch(P, level, cts, gs, keys_h, 0)
    bad = [b for b in range(B) if not np.array_equal(got[b], ref[b])]
    assert not bad, "items differing from the oracle: %s" % bad
    dec = orc.decrypt(P, level, got[0], s_ntt, c["scale"])
    assert rel_err(dec, np.roll(z, -int(offsets[0]))) < 2 ** -20


def test_c5_full_pipeline(lib, orc, full):
    ctx, P = full
    c = S.CONFIGS["C5"]
    B, level = c["batch"], P.L - 1
    announce("C5 full: %d x mul/relin/rescale + 15 rotate-and-sum steps" % B)
    s, s_ntt = secret(orc, P, 5, c["h"])
    n = P.N // 2
    # pair 0: real Q and K activations, N(0,1) scaled by their max to [-1, 1]
    qv = S.normal_values(S.stream(5, "full/Q"), n, 1.0)
    kv = S.normal_values(S.stream(5, "full/K"), n, 1.0)
    qv, kv = qv / np.max(np.abs(qv)), kv / np.max(np.abs(kv))
    a = S.uniform_limbs(S.stream(5, "full/a"), P.q, P.N, lead=(B, 2))
    b = S.uniform_limbs(S.stream(5, "full/b"), P.q, P.N, lead=(B, 2))
    a[0] = encrypt_slots(orc, P, s_ntt, qv.astype(np.complex128), c["scale"], level, 5, "full/encQ")
    b[0] = encrypt_slots(orc, P, s_ntt, kv.astype(np.complex128), c["scale"], level, 5, "full/encK")
    rlk = relin_key(orc, P, s_ntt, 5, tag="full/rlk")
    d_ct = empty_dev((B, 2, level, P.N))
    lib.ckks_mul_relin_rescale(ctx, to_dev(a), to_dev(b), to_dev(rlk), d_ct, B, level)
    steps = c["rotsum_steps"]
    gs = [P.galois(1 << k) for k in range(steps)]
    keys = [galois_key(orc, P, s_ntt, g, 5, "full/rs%d" % k) for k, g in enumerate(gs)]
    d_keys = [to_dev(k) for k in keys]
    lvl = level - 1
    for k in range(steps):
        d_next = empty_dev((B, 2, level, P.N))
        lib.ckks_rotate(ctx, d_ct, d_next, B, lvl, [gs[k]] * B, [d_keys[k]] * B, lib.CKKS_ROT_ACCUMULATE)
        d_ct = d_next
    got = to_host(d_ct)
    for t, m in enumerate(P.q[:level]):
        assert (got[:, :, t, :] < m).all()
    for pair in (0, B // 2, B - 1):
        ref = orc.mul_relin_rescale(P, level, a[pair:pair + 1], b[pair:pair + 1], rlk)[0]
        for k in range(steps):
            ref = orc.rotate(P, lvl, ref, gs[k], keys[k], flags=orc.ROT_ACCUMULATE)
        assert np.array_equal(got[pair], ref), pair
    scale = c["scale"] * c["scale"] / P.q[level]
    dec = orc.decrypt(P, lvl, got[0], s_ntt, scale).real
    total = np.sum(qv * kv)
    assert np.max(np.abs(dec - total)) / np.sum(np.abs(qv * kv)) < 2 ** -12


def test_c4_full_ptmatvec(lib, orc, full):
    ctx, P = full
    c = S.CONFIGS["C4"]
    level, n_in, n_out, n1, n2 = c["level"], c["n_in"], c["n_out"], c["n1"], c["n2"]
    nq = level + 1
    announce("C4 full: ptmatvec %d outputs, %d diagonals at level %d" % (n_out, n_out * n_in * n1 * n2, level))
    torch = torch_cuda()
    x = S.uniform_limbs(S.stream(4, "full/x"), P.q[:nq], P.N, lead=(n_in, 2))
    # 15.7 GB of diagonals: generated and uploaded one output block at a time
    d_diags = torch.empty((n_out, n_in, n2, n1, nq, P.N), dtype=torch.int64, device="cuda")
    kept = {}  # the first and last output blocks' diagonals, for the oracle
    for o in range(n_out):
        blk = S.uniform_limbs(S.stream(o, "full/diag"), P.q[:nq], P.N, lead=(n_in, n2, n1))
        d_diags[o].copy_(torch.from_numpy(blk.view(np.int64)))
        if o in (0, n_out - 1):
            kept[o] = blk
        del blk
    gb = [P.galois(bb) for bb in range(1, n1)]
    gg = [P.galois(n1 * g) for g in range(1, n2)]
    kb = [S.uniform_limbs(S.stream(i, "full/kb"), P.mods, P.N, lead=(P.dnum, 2)) for i in range(n1 - 1)]
    kg = [S.uniform_limbs(S.stream(i, "full/kg"), P.mods, P.N, lead=(P.dnum, 2)) for i in range(n2 - 1)]
    d_y = empty_dev((n_out, 2, level, P.N))
    lib.ckks_ptmatvec(ctx, to_dev(x), n_in, d_diags, n_out, n1, n2, gb, [to_dev(k) for k in kb], gg,
                      [to_dev(k) for k in kg], d_y, level)
    got = to_host(d_y)
    del d_diags
    torch.cuda.empty_cache()
    for t, m in enumerate(P.q[:level]):
        assert (got[:, :, t, :] < m).all()
    # outputs 0 and n_out-1: the first and last diagonal blocks, output slots
    # at both ends of the result buffer
    ref = orc.ptmatvec(P, level, x, np.stack([kept[0], kept[n_out - 1]]), gb, kb, gg, kg)
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[n_out - 1], ref[1])


def test_poly_eval_full(lib, orc, full):
    ctx, P = full
    B, level, scale = 48, P.L - 1, 2.0 ** 54
    coeffs = [1.0, 1.0, 0.5, 1 / 6, 1 / 24, 1 / 120, 1 / 720, 1 / 5040]
    d = len(coeffs) - 1
    announce("poly_eval full: degree %d on %d ciphertexts at N=2^16" % (d, B))
    s, s_ntt = secret(orc, P, 12, 192)
    rlk = relin_key(orc, P, s_ntt, 12, tag="full/pe/rlk")
    cts = S.uniform_limbs(S.stream(12, "full/pe/ct"), P.q, P.N, lead=(B, 2))
    z = S.uniform_slots(S.stream(12, "full/pe/z"), P.N // 2, complex_values=False)
    cts[0] = encrypt_slots(orc, P, s_ntt, z, scale, level, 12, "full/pe/enc")
    out = empty_dev((B, 2, level - d + 1, P.N))
    s_out = lib.ckks_poly_eval(ctx, to_dev(cts), B, level, scale, coeffs, to_dev(rlk), out)
    got = to_host(out)
    for b in (0, B - 1):
        ref, ref_scale = orc.poly_eval(P, level, cts[b:b + 1], scale, coeffs, rlk)
        assert s_out == ref_scale
        assert np.array_equal(got[b], ref[0]), b
    dec = orc.decrypt(P, level - d, got[0], s_ntt, s_out).real
    assert np.max(np.abs(dec - sum(c * z ** k for k, c in enumerate(coeffs)))) < 2 ** -30


def test_av_full_ctmatvec(lib, orc, full):
    ctx, P = full
    c = S.CONFIGS["AV"]
    level, n_in, n_out, n1, n2 = c["level"], c["n_in"], c["n_out"], c["n1"], c["n2"]
    nq = level + 1
    announce("A x V full: ctmatvec %d outputs, %d ciphertext diagonals at level %d"
             % (n_out, n_out * n_in * n1 * n2, level))
    torch = torch_cuda()
    x = S.uniform_limbs(S.stream(7, "full/av/x"), P.q[:nq], P.N, lead=(n_in, 2))
    d_diags = torch.empty((n_out, n_in, n2, n1, 2, nq, P.N), dtype=torch.int64, device="cuda")
    kept = {}  # the first and last output blocks' diagonals, for the oracle
    for o in range(n_out):
        blk = S.uniform_limbs(S.stream(o, "full/av/diag"), P.q[:nq], P.N, lead=(n_in, n2, n1, 2))
        d_diags[o].copy_(torch.from_numpy(blk.view(np.int64)))
        if o in (0, n_out - 1):
            kept[o] = blk
        del blk
    rlk = S.uniform_limbs(S.stream(7, "full/av/rlk"), P.mods, P.N, lead=(P.dnum, 2))
    gb = [P.galois(bb) for bb in range(1, n1)]
    gg = [P.galois(n1 * g) for g in range(1, n2)]
    kb = [S.uniform_limbs(S.stream(i, "full/av/kb"), P.mods, P.N, lead=(P.dnum, 2)) for i in range(n1 - 1)]
    kg = [S.uniform_limbs(S.stream(i, "full/av/kg"), P.mods, P.N, lead=(P.dnum, 2)) for i in range(n2 - 1)]
    d_y = empty_dev((n_out, 2, level, P.N))
    lib.ckks_ctmatvec(ctx, to_dev(x), n_in, d_diags, n_out, n1, n2, to_dev(rlk), gb, [to_dev(k) for k in kb], gg,
                      [to_dev(k) for k in kg], d_y, level)
    got = to_host(d_y)
    del d_diags
    torch.cuda.empty_cache()
    for t, m in enumerate(P.q[:level]):
        assert (got[:, :, t, :] < m).all()
    ref = orc.ctmatvec(P, level, x, np.stack([kept[0], kept[n_out - 1]]), rlk, gb, kb, gg, kg)
    assert np.array_equal(got[0], ref[0])
    assert np.array_equal(got[n_out - 1], ref[1])
