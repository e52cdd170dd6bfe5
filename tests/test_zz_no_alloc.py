"""The allocation-free rotation (ckks_rotate_noalloc) against ckks_rotate,
through the C interface: the same words, bit for bit, on two calls in a row
(the second on a smaller input), at the full workload shape (N = 2^16, 24 + 8
primes, dnum 3), plus its size limit and its checks."""
import numpy as np
import pytest

import ckks_synth as S
from gpu_util import announce, config_pair, empty_dev, make_pair, to_host, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch_cuda()
    import private_rns_ckks_amd as L

    return L


def udev(torch, moduli, N, lead, seed):
    """Uniform residues generated on the device (seeded), [*lead][len(moduli)][N]."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty(tuple(lead) + (len(moduli), N), dtype=torch.int64, device="cuda")
    for i, m in enumerate(moduli):
        out[..., i, :].random_(0, int(m), generator=g)
    return out


def test_noalloc_matches_rotate_full_size(lib, orc):
    torch = torch_cuda()
    c = S.CONFIGS["C3"]
    q = lib.ckks_find_primes(c["log_n"], c["q_bits"], c["L"])
    p = lib.ckks_find_primes(c["log_n"], c["p_bits"], c["K"])
    ref_ctx = lib.Context(c["log_n"], q, p, c["dnum"])
    na_ctx = lib.Context(c["log_n"], q, p, c["dnum"])
    N = 1 << c["log_n"]
    keys = [udev(torch, q + p, N, (c["dnum"], 2), 100 + b) for b in range(3)]
    stream = torch.cuda.current_stream()
    free_before = None
    # call 1: 3 ciphertexts at level 23 (one per chunk: 116 MiB each); call 2:
    # 2 ciphertexts at level 12 with accumulation (two per chunk)
    for call, (batch, level, flags, ks) in enumerate([(3, 23, 0, (1, 4097, 30000)),
                                                      (2, 12, lib.CKKS_ROT_ACCUMULATE, (7, 12345))]):
        announce("noalloc call %d: batch %d level %d flags %d" % (call, batch, level, flags))
        ct = udev(torch, q[: level + 1], N, (batch, 2), 7 + call)
        gs = [pow(5, k, 2 * N) for k in ks]
        out_ref = empty_dev(ct.shape)
        out_na = torch.full(ct.shape, -1, dtype=torch.int64, device="cuda")
        lib.ckks_rotate(ref_ctx, ct, out_ref, batch, level, gs, keys[:batch], flags, stream)
        torch.cuda.synchronize()
        if call == 1:
            free_before = torch.cuda.mem_get_info()[0]
        lib.ckks_rotate_noalloc(na_ctx, ct, out_na, batch, level, gs, keys[:batch], flags, stream)
        torch.cuda.synchronize()
        if call == 1:
            # the second call allocates nothing (its kernels are already loaded)
            assert torch.cuda.mem_get_info()[0] >= free_before - (8 << 20)
        got, ref = to_host(out_na), to_host(out_ref)
        assert np.array_equal(got, ref), "call %d: %d words differ" % (call, int((got != ref).sum()))
        for t, m in enumerate(q[: level + 1]):
            assert (got[:, :, t, :] < m).all()
    ref_ctx.close()
    na_ctx.close()


def test_noalloc_small_params_against_oracle(lib, orc):
    """At N = 2^12 (many ciphertexts per chunk): words equal ckks_rotate's and the oracle's."""
    ctx, P = config_pair(lib, orc, "C3", log_n=12)
    for call, (B, level, flags) in enumerate([(9, 23, 0), (4, 5, 1)]):
        announce("noalloc N=2^12 call %d" % call)
        cts = S.uniform_limbs(S.stream(call, "gpu/na/ct"), P.q[: level + 1], P.N, lead=(B, 2))
        ks = [1, 3, 0, 100, 2047, 5, 9, 11, 13][:B]
        gs = [P.galois(k) for k in ks]
        keys_h = [S.uniform_limbs(S.stream(b, "gpu/na/k"), P.mods, P.N, lead=(P.dnum, 2)) for b in range(B)]
        from gpu_util import to_dev

        keys = [to_dev(k) for k in keys_h]
        d_ct = to_dev(cts)
        a, b = empty_dev(cts.shape), empty_dev(cts.shape)
        lib.ckks_rotate(ctx, d_ct, a, B, level, gs, keys, flags)
        lib.ckks_rotate_noalloc(ctx, d_ct, b, B, level, gs, keys, flags)
        got = to_host(b)
        assert np.array_equal(got, to_host(a))
        assert np.array_equal(got, orc.rotate_batch(P, level, cts, gs, keys_h, orc.ROT_ACCUMULATE if flags else 0))
    ctx.close()


def test_noalloc_limits_and_checks(lib, orc):
    torch = torch_cuda()
    # 48 + 16 primes, dnum 3 at N = 2^16: one ciphertext at level 47 needs
    # N x (48 + 3 x 64 + 2 x 16 + 2 x 48) words = 184 MiB of workspace (more
    # than the 128 MiB scratch); at level 20 (two digits), 84.5 MiB
    q = lib.ckks_find_primes(16, 54, 48)
    p = lib.ckks_find_primes(16, 60, 16)
    ctx = lib.Context(16, q, p, 3)
    N = 1 << 16
    key = torch.zeros((3, 2, 64, N), dtype=torch.int64, device="cuda")
    x = torch.zeros((1, 2, 48, N), dtype=torch.int64, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(lib.CKKSError) as e:
        lib.ckks_rotate_noalloc(ctx, x, y, 1, 47, [5], [key])
    assert e.value.code == lib.CKKS_ERANGE
    assert "scratch" in lib.ckks_last_error()
    lib.ckks_rotate_noalloc(ctx, x[:, :, :21].contiguous(), y[:, :, :21].contiguous(), 1, 20, [5], [key])
    torch.cuda.synchronize()
    # the same argument checks as ckks_rotate
    for args, code in [((1, 48, [5], [key]), lib.CKKS_ERANGE), ((1, 20, [6], [key]), lib.CKKS_EINVAL)]:
        with pytest.raises(lib.CKKSError) as e:
            lib.ckks_rotate_noalloc(ctx, x, y, *args)
        assert e.value.code == code
    with pytest.raises(lib.CKKSError) as e:
        lib.ckks_rotate_noalloc(ctx, x, x, 1, 20, [5], [key])
    assert e.value.code == lib.CKKS_EINVAL
    ctx.close()
