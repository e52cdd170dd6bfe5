"""CPU oracle for the RNS-CKKS rotation hot path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never does, and this package never
imports the GPU library: the two share no code.  Integer arithmetic lives in
``ckks_oracle.c`` (plain ``__int128 %`` modular arithmetic, no fusion, no lazy
reduction); this module adds the ctypes binding and the floating-point
encode/decode, which uses numpy's FFT as a library step.

Conventions (readings of the pages, which give no formula; see the C file's
header for the literature the construction follows):
  * N = 2^log_n, n = N/2 slots; slot j sits at the root zeta^(5^j mod 2N),
    zeta = exp(i*pi/N); its conjugate sits at zeta^(2N - 5^j).
  * Rotation by k slots uses Galois element g = 5^k mod 2N and moves slot
    j+k to slot j (a left shift).
  * Ciphertext primes are the largest primes below 2^bits that are 1 mod 2N
    (descending); special primes likewise below 2^60; psi is the smallest
    primitive 2N-th root of unity of each prime.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ckks_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ROT_ACCUMULATE = 1
NO_RESCALE = 2


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class _Params(ctypes.Structure):
    _fields_ = [
        ("log_n", ctypes.c_int),
        ("L", ctypes.c_int),
        ("K", ctypes.c_int),
        ("dnum", ctypes.c_int),
        ("mod", ctypes.POINTER(ctypes.c_uint64)),
        ("psi", ctypes.POINTER(ctypes.c_uint64)),
    ]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        i64p = ctypes.POINTER(ctypes.c_int64)
        i8p = ctypes.POINTER(ctypes.c_int8)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        pp = ctypes.POINTER(_Params)
        c_int, c_u64, c_u32 = ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32
        sig = {
            "orc_is_prime": (c_int, [c_u64]),
            "orc_gen_primes": (c_int, [c_int, c_int, c_int, u64p]),
            "orc_min_psi": (c_u64, [c_u64, c_int]),
            "orc_ntt_forward": (None, [u64p, c_int, c_u64, c_u64]),
            "orc_ntt_inverse": (None, [u64p, c_int, c_u64, c_u64]),
            "orc_ntt_limbs": (None, [u64p, c_int, c_int, u64p, u64p, c_int]),
            "orc_automorph_coeff": (None, [u64p, u64p, c_int, c_int, u64p, c_u64]),
            "orc_automorph_ntt": (None, [u64p, u64p, c_int, c_int, c_u64]),
            "orc_poly_mul": (None, [u64p, u64p, u64p, c_int, c_int, u64p]),
            "orc_poly_add": (None, [u64p, u64p, u64p, c_int, c_int, u64p]),
            "orc_poly_sub": (None, [u64p, u64p, u64p, c_int, c_int, u64p]),
            "orc_from_signed": (None, [i64p, u64p, c_int, c_int, u64p]),
            "orc_modup": (None, [pp, c_int, c_int, u64p, u64p]),
            "orc_moddown": (None, [pp, c_int, u64p, u64p]),
            "orc_keyswitch": (None, [pp, c_int, u64p, u64p, u64p]),
            "orc_rotate": (None, [pp, c_int, u64p, c_u32, u64p, u64p, ctypes.c_uint]),
            "orc_rotate_batch": (None, [pp, c_int, u64p, c_int, u32p, ctypes.POINTER(u64p), u64p, ctypes.c_uint]),
            "orc_rotate_hoisted": (None, [pp, c_int, u64p, c_int, u32p, ctypes.POINTER(u64p), u64p]),
            "orc_poly_eval": (c_int, [pp, c_int, u64p, c_int, ctypes.c_double, ctypes.POINTER(ctypes.c_double), c_int,
                                      u64p, u64p, ctypes.POINTER(ctypes.c_double)]),
            "orc_poly_eval_tree": (c_int, [pp, c_int, u64p, c_int, ctypes.c_double, ctypes.POINTER(ctypes.c_double),
                                           c_int, u64p, u64p, ctypes.POINTER(ctypes.c_double)]),
            "orc_rescale": (c_int, [pp, c_int, u64p, u64p]),
            "orc_tensor": (None, [pp, c_int, u64p, u64p, u64p]),
            "orc_mul_relin_rescale": (c_int, [pp, c_int, u64p, u64p, u64p, u64p, c_int, ctypes.c_uint]),
            "orc_ptmatvec": (c_int, [pp, c_int, u64p, c_int, u64p, c_int, c_int, c_int, u32p, ctypes.POINTER(u64p),
                                     u32p, ctypes.POINTER(u64p), u64p, ctypes.c_uint, c_int, c_int]),
            "orc_ctmatvec": (c_int, [pp, c_int, u64p, c_int, u64p, c_int, c_int, c_int, u64p, u32p,
                                     ctypes.POINTER(u64p), u32p, ctypes.POINTER(u64p), u64p, ctypes.c_uint, c_int,
                                     c_int]),
            "orc_secret_ntt": (None, [pp, i8p, u64p]),
            "orc_make_switch_key": (None, [pp, u64p, u64p, u64p, i64p, u64p]),
            "orc_encrypt": (None, [pp, c_int, u64p, u64p, u64p, i64p, u64p]),
            "orc_decrypt_coeff": (None, [pp, c_int, u64p, u64p, u64p]),
            "orc_num_threads": (c_int, []),
            "orc_set_num_threads": (None, [c_int]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _u64(a):
    assert a.dtype == np.uint64 and a.flags["C_CONTIGUOUS"], "expected contiguous uint64"
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))


def _i64(a):
    assert a.dtype == np.int64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _arr(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint64))


def _ptr_array(arrs):
    u64p = ctypes.POINTER(ctypes.c_uint64)
    return (u64p * len(arrs))(*[_u64(a) for a in arrs])


# ---------------------------------------------------------------------------
# Parameters
# ---------------------------------------------------------------------------

def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP thread count of the oracle's parallel loops."""
    lib().orc_set_num_threads(int(n))


def is_prime(n: int) -> bool:
    return bool(lib().orc_is_prime(int(n)))


def gen_primes(log_n: int, bits: int, count: int) -> list:
    out = np.zeros(count, dtype=np.uint64)
    got = lib().orc_gen_primes(log_n, bits, count, _u64(out))
    if got != count:
        raise ValueError("not enough primes")
    return [int(v) for v in out]


def min_psi(m: int, log_n: int) -> int:
    return int(lib().orc_min_psi(int(m), log_n))


@dataclass
class Params:
    """RNS-CKKS parameters: N = 2^log_n, ciphertext primes q (L of them,
    q_0 first), special primes p (K), gadget digit count dnum."""

    log_n: int
    q: list
    p: list
    dnum: int
    psi: list = field(default=None)

    def __post_init__(self):
        self.q = [int(v) for v in self.q]
        self.p = [int(v) for v in self.p]
        if self.psi is None:
            self.psi = [min_psi(m, self.log_n) for m in self.q + self.p]
        self._mods = _arr(self.q + self.p)
        self._psis = _arr(self.psi)
        self._c = _Params(self.log_n, len(self.q), len(self.p), self.dnum,
                          _u64(self._mods), _u64(self._psis))

    @classmethod
    def generate(cls, log_n: int, L: int, q_bits: int, K: int, p_bits: int, dnum: int) -> "Params":
        return cls(log_n, gen_primes(log_n, q_bits, L), gen_primes(log_n, p_bits, K) if K else [], dnum)

    @property
    def N(self) -> int:
        return 1 << self.log_n

    @property
    def L(self) -> int:
        return len(self.q)

    @property
    def K(self) -> int:
        return len(self.p)

    @property
    def alpha(self) -> int:
        return -(-self.L // self.dnum)

    @property
    def mods(self) -> list:
        return self.q + self.p

    def beta(self, level: int) -> int:
        return -(-(level + 1) // self.alpha)

    def ext_mods(self, level: int) -> list:
        return self.q[: level + 1] + self.p

    def ref(self):
        return ctypes.byref(self._c)

    def galois(self, k: int) -> int:
        """Galois element of a left rotation by k slots."""
        n = self.N // 2
        return pow(5, k % n, 2 * self.N)


# ---------------------------------------------------------------------------
# NTT and automorphism
# ---------------------------------------------------------------------------

def ntt(a, mods, psis, log_n, inverse=False):
    """Transform every limb of a[..., nlimb, N]; limb i uses mods[i], psis[i]."""
    a = _arr(a).copy()
    nl = a.shape[-2]
    flat = a.reshape(-1, nl, a.shape[-1])
    m, s = _arr(mods), _arr(psis)
    for blk in flat:
        lib().orc_ntt_limbs(_u64(blk), nl, log_n, _u64(m), _u64(s), int(inverse))
    return a


def ntt_params(P: Params, a, limb_begin=0, inverse=False):
    nl = np.asarray(a).shape[-2]
    return ntt(a, P.mods[limb_begin: limb_begin + nl], P.psi[limb_begin: limb_begin + nl], P.log_n, inverse)


def automorph_coeff(a, mods, log_n, g):
    a = _arr(a)
    out = np.empty_like(a)
    nl = a.shape[-2]
    m = _arr(mods)
    for src, dst in zip(a.reshape(-1, nl, a.shape[-1]), out.reshape(-1, nl, a.shape[-1])):
        lib().orc_automorph_coeff(_u64(src), _u64(dst), nl, log_n, _u64(m), int(g))
    return out


def automorph_ntt(a, log_n, g):
    a = _arr(a)
    out = np.empty_like(a)
    nl = a.shape[-2]
    for src, dst in zip(a.reshape(-1, nl, a.shape[-1]), out.reshape(-1, nl, a.shape[-1])):
        lib().orc_automorph_ntt(_u64(src), _u64(dst), nl, log_n, int(g))
    return out


# ---------------------------------------------------------------------------
# Basis conversion, key switching and the operations built on it
# ---------------------------------------------------------------------------

def modup(P: Params, level: int, j: int, x_coeff):
    x = _arr(x_coeff)
    out = np.empty((level + 1 + P.K, P.N), dtype=np.uint64)
    lib().orc_modup(P.ref(), level, j, _u64(x), _u64(out))
    return out


def moddown(P: Params, level: int, acc_ntt):
    a = _arr(acc_ntt)
    out = np.empty((level + 1, P.N), dtype=np.uint64)
    lib().orc_moddown(P.ref(), level, _u64(a), _u64(out))
    return out


def keyswitch(P: Params, level: int, d, evk):
    d, evk = _arr(d), _arr(evk)
    assert evk.shape == (P.dnum, 2, P.L + P.K, P.N)
    out = np.empty((2, level + 1, P.N), dtype=np.uint64)
    lib().orc_keyswitch(P.ref(), level, _u64(d), _u64(evk), _u64(out))
    return out


def rotate(P: Params, level: int, ct, g: int, evk, flags: int = 0):
    ct = _arr(ct)
    out = np.empty_like(ct)
    lib().orc_rotate(P.ref(), level, _u64(ct), int(g), _u64(_arr(evk)), _u64(out), flags)
    return out


def rotate_batch(P: Params, level: int, cts, gs, evks, flags: int = 0):
    cts = _arr(cts)
    B = cts.shape[0]
    out = np.empty_like(cts)
    evks = [_arr(e) for e in evks]
    g = np.ascontiguousarray(np.asarray(gs, dtype=np.uint32))
    lib().orc_rotate_batch(P.ref(), level, _u64(cts), B, g.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                           _ptr_array(evks), _u64(out), flags)
    return out


def rotate_hoisted(P: Params, level: int, ct, gs, evks):
    """Rotations of one ciphertext by every element of gs sharing one basis
    extension; returns [len(gs)][2][l+1][N]."""
    ct = _arr(ct)
    R = len(gs)
    out = np.empty((R,) + ct.shape, dtype=np.uint64)
    evks = [_arr(e) for e in evks]
    g = np.ascontiguousarray(np.asarray(gs, dtype=np.uint32))
    lib().orc_rotate_hoisted(P.ref(), level, _u64(ct), R, g.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)),
                             _ptr_array(evks), _u64(out))
    return out


def rescale(P: Params, level: int, ct):
    ct = _arr(ct)
    out = np.empty((2, level, P.N), dtype=np.uint64)
    rc = lib().orc_rescale(P.ref(), level, _u64(ct), _u64(out))
    if rc != 0:
        raise ValueError("rescale at level 0")
    return out


def tensor(P: Params, level: int, a, b):
    out = np.empty((3, level + 1, P.N), dtype=np.uint64)
    lib().orc_tensor(P.ref(), level, _u64(_arr(a)), _u64(_arr(b)), _u64(out))
    return out


def mul_relin_rescale(P: Params, level: int, a, b, rlk, flags: int = 0):
    a, b = _arr(a), _arr(b)
    B = a.shape[0]
    lo = level + 1 if flags & NO_RESCALE else level
    out = np.empty((B, 2, lo, P.N), dtype=np.uint64)
    rc = lib().orc_mul_relin_rescale(P.ref(), level, _u64(a), _u64(b), _u64(_arr(rlk)), _u64(out), B, flags)
    if rc != 0:
        raise ValueError("rescale at level 0")
    return out


def poly_eval(P: Params, level: int, cts, scale: float, coeffs, rlk):
    """p(x) = sum_k coeffs[k] x^k on [B][2][l+1][N] ciphertexts by Horner's
    rule; returns ([B][2][l-d+1][N], output scale)."""
    cts = _arr(cts)
    B = cts.shape[0]
    d = len(coeffs) - 1
    out = np.empty((B, 2, level - d + 1, P.N), dtype=np.uint64)
    c = (ctypes.c_double * len(coeffs))(*[float(v) for v in coeffs])
    s = ctypes.c_double(0.0)
    rc = lib().orc_poly_eval(P.ref(), level, _u64(cts), B, float(scale), c, d, _u64(_arr(rlk)), _u64(out),
                             ctypes.byref(s))
    if rc == -2:
        raise ValueError("degree must be 1..level")
    if rc == -3:
        raise ValueError("a rounded constant reaches 2^62")
    return out, s.value


def tree_depth(degree: int) -> int:
    """Levels consumed by poly_eval_tree: ceil(log2(degree + 1))."""
    return degree.bit_length()


def poly_eval_tree(P: Params, level: int, cts, scale: float, coeffs, rlk):
    """p(x) = sum_k coeffs[k] x^k on [B][2][l+1][N] ciphertexts by the
    power-basis baby-step / giant-step split with scales fixed top-down
    (depth ceil(log2(d + 1))); returns ([B][2][l - depth + 1][N], output
    scale = scale)."""
    cts = _arr(cts)
    B = cts.shape[0]
    d = len(coeffs) - 1
    lo = level - tree_depth(d) + 1 if d >= 1 else 1
    out = np.empty((B, 2, max(lo, 1), P.N), dtype=np.uint64)
    c = (ctypes.c_double * len(coeffs))(*[float(v) for v in coeffs])
    s = ctypes.c_double(0.0)
    rc = lib().orc_poly_eval_tree(P.ref(), level, _u64(cts), B, float(scale), c, d, _u64(_arr(rlk)), _u64(out),
                                  ctypes.byref(s))
    if rc == -2:
        raise ValueError("degree must be 1..64 and the level at least ceil(log2(degree + 1))")
    if rc == -3:
        raise ValueError("a rounded constant reaches 2^62")
    return out, s.value


def ptmatvec(P: Params, level: int, x, diags, g_baby, evk_baby, g_giant, evk_giant, flags: int = 0,
             o_range=None):
    """BSGS plaintext matvec; diags: [n_out][n_in][n2][n1][l+1][N].  Returns
    y [n_out][2][l or l+1][N]; with o_range=(a, b) only outputs a..b-1 are
    computed (others are left zero)."""
    x, diags = _arr(x), _arr(diags)
    n_out, n_in, n2, n1 = diags.shape[:4]
    lo = level + 1 if flags & NO_RESCALE else level
    y = np.zeros((n_out, 2, lo, P.N), dtype=np.uint64)
    gb = np.ascontiguousarray(np.asarray(list(g_baby) + [0], dtype=np.uint32))
    gg = np.ascontiguousarray(np.asarray(list(g_giant) + [0], dtype=np.uint32))
    eb = [_arr(e) for e in evk_baby] or [np.zeros(1, dtype=np.uint64)]
    eg = [_arr(e) for e in evk_giant] or [np.zeros(1, dtype=np.uint64)]
    a, b = o_range if o_range is not None else (0, n_out)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    rc = lib().orc_ptmatvec(P.ref(), level, _u64(x), n_in, _u64(diags), n_out, n1, n2,
                            gb.ctypes.data_as(u32p), _ptr_array(eb), gg.ctypes.data_as(u32p), _ptr_array(eg),
                            _u64(y), flags, a, b)
    if rc != 0:
        raise ValueError("rescale at level 0")
    return y


def ctmatvec(P: Params, level: int, x, diags, rlk, g_baby, evk_baby, g_giant, evk_giant, flags: int = 0,
             o_range=None):
    """BSGS matvec with encrypted weights (the A x V product of attention);
    diags: [n_out][n_in][n2][n1][2][l+1][N] ciphertexts, rlk the s^2 -> s key.
    Tensor products of a giant-step group are summed and relinearised once.
    Returns y [n_out][2][l or l+1][N]; o_range as in ptmatvec."""
    x, diags, rlk = _arr(x), _arr(diags), _arr(rlk)
    n_out, n_in, n2, n1 = diags.shape[:4]
    lo = level + 1 if flags & NO_RESCALE else level
    y = np.zeros((n_out, 2, lo, P.N), dtype=np.uint64)
    gb = np.ascontiguousarray(np.asarray(list(g_baby) + [0], dtype=np.uint32))
    gg = np.ascontiguousarray(np.asarray(list(g_giant) + [0], dtype=np.uint32))
    eb = [_arr(e) for e in evk_baby] or [np.zeros(1, dtype=np.uint64)]
    eg = [_arr(e) for e in evk_giant] or [np.zeros(1, dtype=np.uint64)]
    a, b = o_range if o_range is not None else (0, n_out)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    rc = lib().orc_ctmatvec(P.ref(), level, _u64(x), n_in, _u64(diags), n_out, n1, n2, _u64(rlk),
                            gb.ctypes.data_as(u32p), _ptr_array(eb), gg.ctypes.data_as(u32p), _ptr_array(eg),
                            _u64(y), flags, a, b)
    if rc != 0:
        raise ValueError("rescale at level 0")
    return y


# ---------------------------------------------------------------------------
# Keys, encryption, decryption
# ---------------------------------------------------------------------------

def secret_ntt(P: Params, s_coeff):
    s = np.ascontiguousarray(np.asarray(s_coeff, dtype=np.int8))
    out = np.empty((P.L + P.K, P.N), dtype=np.uint64)
    lib().orc_secret_ntt(P.ref(), s.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), _u64(out))
    return out


def switch_key(P: Params, s_from_ntt, s_ntt, a, e):
    """a: uniform [dnum][L+K][N] (NTT form); e: signed errors [dnum][N]."""
    a = _arr(a)
    e = np.ascontiguousarray(np.asarray(e, dtype=np.int64))
    assert a.shape == (P.dnum, P.L + P.K, P.N) and e.shape == (P.dnum, P.N)
    out = np.empty((P.dnum, 2, P.L + P.K, P.N), dtype=np.uint64)
    lib().orc_make_switch_key(P.ref(), _u64(_arr(s_from_ntt)), _u64(_arr(s_ntt)), _u64(a), _i64(e), _u64(out))
    return out


def galois_key(P: Params, s_ntt, g: int, a, e):
    """Key switching from tau_g(s) back to s."""
    return switch_key(P, automorph_ntt(s_ntt, P.log_n, g), s_ntt, a, e)


def relin_key(P: Params, s_ntt, a, e):
    """Key switching from s^2 back to s."""
    s2 = np.empty_like(_arr(s_ntt))
    lib().orc_poly_mul(_u64(_arr(s_ntt)), _u64(_arr(s_ntt)), _u64(s2), P.L + P.K, P.log_n, _u64(P._mods))
    return switch_key(P, s2, s_ntt, a, e)


def from_signed(P: Params, c, nlimb: int):
    c = np.ascontiguousarray(np.asarray(c, dtype=np.int64))
    out = np.empty((nlimb, P.N), dtype=np.uint64)
    lib().orc_from_signed(_i64(c), _u64(out), nlimb, P.log_n, _u64(P._mods))
    return out


def encrypt(P: Params, level: int, pt_ntt, s_ntt, a, e):
    out = np.empty((2, level + 1, P.N), dtype=np.uint64)
    lib().orc_encrypt(P.ref(), level, _u64(_arr(pt_ntt)), _u64(_arr(s_ntt)), _u64(_arr(a)),
                      _i64(np.ascontiguousarray(np.asarray(e, dtype=np.int64))), _u64(out))
    return out


def decrypt_coeff(P: Params, level: int, ct, s_ntt):
    out = np.empty((level + 1, P.N), dtype=np.uint64)
    lib().orc_decrypt_coeff(P.ref(), level, _u64(_arr(ct)), _u64(_arr(s_ntt)), _u64(out))
    return out


# ---------------------------------------------------------------------------
# CRT and the canonical embedding (encode / decode)
# ---------------------------------------------------------------------------

def crt_centered(limbs, mods):
    """Python-int CRT of limbs [k][N] (residues modulo mods), lifted to the
    centered range [-(Q-1)/2, (Q-1)/2].  Returns an object array of ints."""
    mods = [int(m) for m in mods]
    Q = 1
    for m in mods:
        Q *= m
    acc = np.zeros(np.asarray(limbs).shape[-1], dtype=object)
    for x, m in zip(np.asarray(limbs), mods):
        Qi = Q // m
        c = pow(Qi % m, -1, m)
        acc = acc + ((x.astype(object) * c) % m) * Qi
    acc = acc % Q
    half = Q // 2
    return np.where(acc > half, acc - Q, acc)


def slot_exponents(N: int) -> np.ndarray:
    """e_j = 5^j mod 2N for the N/2 slots."""
    n = N // 2
    e = np.empty(n, dtype=np.int64)
    v = 1
    for j in range(n):
        e[j] = v
        v = v * 5 % (2 * N)
    return e


def encode_coeffs(z, N: int, scale: float) -> np.ndarray:
    """Integer coefficients m with m(zeta^(5^j)) ~= scale * z_j (rounded to nearest)."""
    z = np.asarray(z, dtype=np.complex128)
    n = N // 2
    assert z.shape == (n,)
    e = slot_exponents(N)
    Z = np.zeros(N, dtype=np.complex128)
    Z[(e - 1) // 2] = scale * z
    Z[(2 * N - e - 1) // 2] = np.conj(scale * z)
    k = np.arange(N)
    zeta_neg = np.exp(-1j * np.pi * k / N)
    m = (zeta_neg * np.fft.fft(Z)).real / N
    return np.rint(m).astype(np.int64)


def decode_coeffs(m, N: int, scale: float) -> np.ndarray:
    """Slots z_j = m(zeta^(5^j)) / scale from real (float or int) coefficients m."""
    m = np.asarray(m, dtype=np.float64)
    k = np.arange(N)
    c = m * np.exp(1j * np.pi * k / N)
    ev = np.fft.ifft(c) * N
    e = slot_exponents(N)
    return ev[(e - 1) // 2] / scale


def encode(P: Params, z, scale: float, level: int):
    """Plaintext in NTT form on limbs q_0..q_level."""
    m = encode_coeffs(z, P.N, scale)
    return ntt_params(P, from_signed(P, m, level + 1))


def decode_limbs(P: Params, coeff_limbs, scale: float, level: int):
    x = crt_centered(coeff_limbs, P.q[: level + 1])
    return decode_coeffs(np.array([float(v) for v in x]), P.N, scale)


def decrypt(P: Params, level: int, ct, s_ntt, scale: float):
    return decode_limbs(P, decrypt_coeff(P, level, ct, s_ntt), scale, level)
