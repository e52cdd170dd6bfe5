"""Helpers for the GPU parity tests: move uint64 words between numpy and the
device, and build a library context for a workload recipe.  The library's
primes come from its own search (ckks_find_primes); tests check they equal
the oracle's."""
from __future__ import annotations

import numpy as np
import pytest

import ckks_synth as S

try:  # imported at collection so the first test does not pay for it
    import torch as _torch  # noqa: F401
except ImportError:  # pragma: no cover
    _torch = None


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(arr):
    torch = torch_cuda()
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.uint64))
    return torch.from_numpy(a.view(np.int64)).to("cuda")


def empty_dev(shape):
    torch = torch_cuda()
    return torch.empty(tuple(shape), dtype=torch.int64, device="cuda")


def misaligned_dev(shape):
    """A device tensor of `shape` whose data starts 8 bytes past a 16-byte boundary."""
    torch = torch_cuda()
    n = int(np.prod(shape))
    buf = torch.empty(n + 2, dtype=torch.int64, device="cuda")
    return buf[1:1 + n].view(tuple(shape))


def to_host(t):
    torch = torch_cuda()
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint64)


def lib_params(lib, log_n, L, q_bits, K, p_bits, dnum):
    q = lib.ckks_find_primes(log_n, q_bits, L)
    p = lib.ckks_find_primes(log_n, p_bits, K) if K else []
    return q, p, dnum


def make_pair(lib, orc, log_n, L, q_bits, K, p_bits, dnum):
    """(library Context, oracle Params) for one parameter set, primes found independently."""
    q, p, dnum = lib_params(lib, log_n, L, q_bits, K, p_bits, dnum)
    P = orc.Params.generate(log_n, L, q_bits, K, p_bits, dnum)
    assert P.q == q and P.p == p
    ctx = lib.Context(log_n, q, p, dnum)
    assert ctx.psi == P.psi
    return ctx, P


def config_pair(lib, orc, name, log_n=None):
    c = S.CONFIGS[name]
    return make_pair(lib, orc, log_n or c["log_n"], c["L"], c["q_bits"], c["K"], c["p_bits"], c["dnum"])


def announce(msg):
    print("[gpu-case] " + msg, flush=True)
