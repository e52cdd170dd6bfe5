"""Test-side helpers: build oracle parameters, keys and ciphertexts from the
seeded generators.  Everything here calls the oracle or ckks_synth only."""
from __future__ import annotations

import numpy as np

import ckks_synth as S


def params(orc, log_n, L, q_bits, K, p_bits, dnum):
    return orc.Params.generate(log_n, L, q_bits, K, p_bits, dnum)


def config_params(orc, name, log_n=None):
    c = S.CONFIGS[name]
    return orc.Params.generate(log_n or c["log_n"], c["L"], c["q_bits"], c["K"], c["p_bits"], c["dnum"])


def secret(orc, P, seed, h):
    s = S.ternary_secret(S.stream(seed, "sk"), P.N, h)
    return s, orc.secret_ntt(P, s)


def switch_key_inputs(P, seed, tag, sigma=3.2, zero_error=False):
    a = S.uniform_limbs(S.stream(seed, tag + "/a"), P.mods, P.N, lead=(P.dnum,))
    if zero_error:
        e = np.zeros((P.dnum, P.N), dtype=np.int64)
    else:
        e = S.rounded_gaussian(S.stream(seed, tag + "/e"), (P.dnum, P.N), sigma)
    return a, e


def galois_key(orc, P, s_ntt, g, seed, tag, zero_error=False):
    a, e = switch_key_inputs(P, seed, tag, zero_error=zero_error)
    return orc.galois_key(P, s_ntt, g, a, e)


def relin_key(orc, P, s_ntt, seed, tag="rlk", zero_error=False):
    a, e = switch_key_inputs(P, seed, tag, zero_error=zero_error)
    return orc.relin_key(P, s_ntt, a, e)


def encrypt_slots(orc, P, s_ntt, z, scale, level, seed, tag, sigma=3.2):
    pt = orc.encode(P, z, scale, level)
    a = S.uniform_limbs(S.stream(seed, tag + "/a"), P.q[: level + 1], P.N)
    e = S.rounded_gaussian(S.stream(seed, tag + "/e"), P.N, sigma)
    return orc.encrypt(P, level, pt, s_ntt, a, e)


def rel_err(got, ref):
    return float(np.max(np.abs(np.asarray(got) - np.asarray(ref))) / np.max(np.abs(np.asarray(ref))))


def centered_coeffs(orc, limbs_coeff, mods):
    """Python-int centered CRT values of coefficient-form limbs."""
    return orc.crt_centered(limbs_coeff, mods)
