"""Host-side checks of the C interface (no GPU work): the library loads, it
exports every entry point include/ckks.h declares, the prime search agrees
with the oracle's, and parameter validation rejects bad sets with the
documented codes."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import private_rns_ckks_amd as P

    return P


def declared_functions(header=None):
    """Functions declared by include/<header>, or by every header in include/."""
    inc = os.path.join(ROOT, "include")
    files = [header] if header else sorted(f for f in os.listdir(inc) if f.endswith(".h"))
    names = set()
    for f in files:
        text = open(os.path.join(inc, f)).read()
        names |= set(re.findall(r"^\s*(?:int|const char\*)\s+(ckks_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_hot_path_calls():
    names = declared_functions("ckks.h")
    for n in ["ckks_ntt", "ckks_automorph", "ckks_keyswitch", "ckks_rotate", "ckks_ptmatvec",
              "ckks_mul_relin_rescale"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib.lib(), n), n
    assert sorted(lib.EXPORTED) == names


def test_find_primes_matches_oracle(lib, orc):
    for log_n, bits, count in [(12, 30, 4), (12, 60, 1), (16, 54, 24), (16, 60, 8), (10, 40, 5), (12, 62, 3),
                               (16, 61, 2)]:
        assert lib.ckks_find_primes(log_n, bits, count) == orc.gen_primes(log_n, bits, count)


def test_find_primes_errors(lib):
    with pytest.raises(lib.CKKSError) as e:
        lib.ckks_find_primes(16, 17, 1000)
    assert e.value.code == lib.CKKS_EPARAM


def c3(lib):
    return 16, lib.ckks_find_primes(16, 54, 24), lib.ckks_find_primes(16, 60, 8), 3


def test_params_validate_accepts_configs(lib, orc):
    assert lib.ckks_params_validate(*c3(lib)) == lib.CKKS_OK
    q, p = lib.ckks_find_primes(12, 30, 4), lib.ckks_find_primes(12, 60, 1)
    assert lib.ckks_params_validate(12, q, p, 4) == lib.CKKS_OK
    psi = [orc.min_psi(m, 12) for m in q + p]
    assert lib.ckks_params_validate(12, q, p, 4, psi) == lib.CKKS_OK


def test_params_validate_rejects(lib):
    log_n, q, p, dnum = c3(lib)
    E = lib.CKKS_EPARAM
    assert lib.ckks_params_validate(17, q, p, dnum) == E            # N too large
    assert lib.ckks_params_validate(9, q, p, dnum) == E             # N too small
    assert lib.ckks_params_validate(log_n, q, p[:7], dnum) == E     # K != alpha
    assert lib.ckks_params_validate(log_n, q, p, 0) == E            # dnum 0
    assert lib.ckks_params_validate(log_n, q, p, 25) == E           # dnum > L
    assert lib.ckks_params_validate(log_n, [q[0] + 2] + q[1:], p, dnum) == E  # not 1 mod 2N
    assert lib.ckks_params_validate(log_n, [q[0] + (2 << log_n)] + q[1:], p, dnum) == E  # composite (or 1 mod 2N but not prime)
    assert lib.ckks_params_validate(log_n, [q[1]] + q[1:], p, dnum) == E      # duplicate
    assert lib.ckks_params_validate(log_n, q, p, dnum, [2] * 32) == E         # bad psi
    assert lib.ckks_params_validate(log_n, [], p, dnum) == E
    assert "n_p" in lib.ckks_last_error() or lib.ckks_last_error() != ""
    # primes up to 2^62 are accepted, 2^62 and above rejected
    wq, wp = lib.ckks_find_primes(12, 62, 6), lib.ckks_find_primes(12, 61, 2)
    assert lib.ckks_params_validate(12, wq, wp, 3) == lib.CKKS_OK
    big = next(m for m in range(2 ** 62 + 1, 2 ** 62 + (2 << 12) * 4000, 2 << 12) if pow(3, m - 1, m) == 1)
    assert lib.ckks_params_validate(12, [big] + wq[1:], wp, 3) == E
    assert "2^62" in lib.ckks_last_error()


def test_strerror(lib):
    assert lib.ckks_strerror(0) == "ok"
    for code in range(-6, 0):
        assert lib.ckks_strerror(code) not in ("ok", "unknown status")
