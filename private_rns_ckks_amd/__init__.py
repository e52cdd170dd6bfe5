"""Python binding of libckks_mi355x.so, the gfx950 RNS-CKKS rotation hot path.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Device buffers are torch tensors of dtype int64 (reinterpreted as
uint64 words, contiguous, on a ROCm device); streams are torch.cuda.Stream
objects (or None for the current stream).  The function names are those of
the C interface in include/ckks.h, which documents layouts and semantics.

Importing this package loads the compiled library and raises if it is
missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libckks_mi355x.so")

CKKS_OK = 0
CKKS_EINVAL = -1
CKKS_ERANGE = -2
CKKS_ENOMEM = -3
CKKS_EHIP = -4
CKKS_EPARAM = -5
CKKS_EINTERNAL = -6
CKKS_ROT_ACCUMULATE = 1
CKKS_NO_RESCALE = 2

EXPORTED = [
    "ckks_find_primes", "ckks_params_validate", "ckks_strerror", "ckks_last_error",
    "ckks_ctx_create", "ckks_ctx_destroy", "ckks_ctx_psi",
    "ckks_ntt", "ckks_automorph", "ckks_keyswitch", "ckks_rotate", "ckks_rotate_noalloc", "ckks_rotate_hoisted",
    "ckks_rescale",
    "ckks_mul_relin_rescale", "ckks_poly_eval", "ckks_poly_eval_tree", "ckks_ptmatvec", "ckks_ctmatvec", "ckks_trace_begin",
    "ckks_trace_end", "ckks_probe_list", "ckks_probe_rate",
]

# Kernel whose launches take the largest share of a rotation batch (by
# rocprofv3 time): the ciphertext-prime inner product fused with the final
# combination.
DOMINANT_KERNEL = "comb_ip"


class CKKSError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s failed: %s (%d): %s" % (where, _lib.ckks_strerror(code).decode(), code,
                                                    _lib.ckks_last_error().decode()))


class ckks_trace_stats(ctypes.Structure):
    _fields_ = [("launches", ctypes.c_int32), ("total_ms", ctypes.c_double), ("work_units", ctypes.c_double)]


class ckks_params(ctypes.Structure):
    _fields_ = [
        ("log_n", ctypes.c_uint32),
        ("n_q", ctypes.c_uint32),
        ("n_p", ctypes.c_uint32),
        ("dnum", ctypes.c_uint32),
        ("q", ctypes.POINTER(ctypes.c_uint64)),
        ("p", ctypes.POINTER(ctypes.c_uint64)),
        ("psi", ctypes.POINTER(ctypes.c_uint64)),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libckks_mi355x.so is not built (%s); run __graft_entry__.build() or "
                          "python private_rns_ckks_amd/build.py" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, u64p, u32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint32)
    i, u32 = ctypes.c_int, ctypes.c_uint32
    pp = ctypes.POINTER(vp)
    sig = {
        "ckks_find_primes": (i, [u32, u32, u32, u64p]),
        "ckks_params_validate": (i, [ctypes.POINTER(ckks_params)]),
        "ckks_strerror": (ctypes.c_char_p, [i]),
        "ckks_last_error": (ctypes.c_char_p, []),
        "ckks_ctx_create": (i, [ctypes.POINTER(ckks_params), i, ctypes.POINTER(vp)]),
        "ckks_ctx_destroy": (i, [vp]),
        "ckks_ctx_psi": (i, [vp, u64p]),
        "ckks_ntt": (i, [vp, vp, i, i, i, i, vp]),
        "ckks_automorph": (i, [vp, vp, vp, i, i, u32, i, vp]),
        "ckks_keyswitch": (i, [vp, vp, vp, vp, i, vp]),
        "ckks_rotate": (i, [vp, vp, vp, i, i, u32p, pp, ctypes.c_uint, vp]),
        "ckks_rotate_noalloc": (i, [vp, vp, vp, i, i, u32p, pp, ctypes.c_uint, vp]),
        "ckks_rotate_hoisted": (i, [vp, vp, i, i, i, u32p, pp, vp, vp]),
        "ckks_rescale": (i, [vp, vp, vp, i, i, vp]),
        "ckks_mul_relin_rescale": (i, [vp, vp, vp, vp, vp, i, i, ctypes.c_uint, vp]),
        "ckks_poly_eval": (i, [vp, vp, i, i, ctypes.c_double, ctypes.POINTER(ctypes.c_double), i, vp, vp,
                               ctypes.POINTER(ctypes.c_double), vp]),
        "ckks_poly_eval_tree": (i, [vp, vp, i, i, ctypes.c_double, ctypes.POINTER(ctypes.c_double), i, vp, vp,
                                    ctypes.POINTER(ctypes.c_double), vp]),
        "ckks_ptmatvec": (i, [vp, vp, i, vp, i, i, i, u32p, pp, u32p, pp, vp, i, ctypes.c_uint, vp]),
        "ckks_ctmatvec": (i, [vp, vp, i, vp, i, i, i, vp, u32p, pp, u32p, pp, vp, i, ctypes.c_uint, vp]),
        "ckks_trace_begin": (i, [vp, ctypes.c_char_p]),
        "ckks_trace_end": (i, [vp, ctypes.POINTER(ckks_trace_stats)]),
        "ckks_probe_list": (i, [ctypes.c_char_p, i]),
        "ckks_probe_rate": (i, [i, ctypes.c_char_p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def lib():
    return _lib


def _check(rc, where):
    if rc != CKKS_OK:
        raise CKKSError(rc, where)


class ArgumentError(ValueError):
    """A tensor or list argument does not fit the call (raised on the host,
    before the library is called, so no launch ever sees it)."""


def _ptr(t):
    """Device pointer of a contiguous int64 torch tensor (or None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ArgumentError("tensor must be contiguous")
    if t.element_size() != 8:
        raise ArgumentError("tensor must hold 64-bit words")
    return ctypes.c_void_p(t.data_ptr())


def _dev(ctx, t, words, what, optional=False):
    """Pointer of a device tensor the call reads or writes `words` 64-bit
    words of: checked to be a contiguous 8-byte tensor on the context's
    device holding at least that many words.  `words` None skips the size
    check (the library rejects the call's level or count itself)."""
    if t is None:
        if optional:
            return None
        raise ArgumentError("%s is None" % what)
    if not getattr(t, "is_cuda", False):
        raise ArgumentError("%s must be a device tensor" % what)
    if t.device.index is not None and t.device.index != ctx.device:
        raise ArgumentError("%s is on device %d, the context on device %d" % (what, t.device.index, ctx.device))
    ptr = _ptr(t)
    if words is not None and t.numel() < words:
        raise ArgumentError("%s holds %d words; the call touches %d" % (what, t.numel(), words))
    return ptr


def _count(seq, n, what):
    if len(seq) != n:
        raise ArgumentError("%s has %d entries; the call needs %d" % (what, len(seq), n))


def _stream(stream):
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _u64_array(vals):
    return (ctypes.c_uint64 * len(vals))(*[int(v) for v in vals])


def ckks_find_primes(log_n, bits, count):
    out = (ctypes.c_uint64 * count)()
    _check(_lib.ckks_find_primes(log_n, bits, count, out), "ckks_find_primes")
    return [int(v) for v in out]


def _params_struct(log_n, q, p, dnum, psi=None):
    qa, pa = _u64_array(q), _u64_array(p) if p else None
    sa = _u64_array(psi) if psi is not None else None
    st = ckks_params(log_n, len(q), len(p), dnum, qa, pa, sa)
    st._keep = (qa, pa, sa)
    return st


def ckks_params_validate(log_n, q, p, dnum, psi=None):
    """Returns the status code (0 = valid)."""
    return _lib.ckks_params_validate(ctypes.byref(_params_struct(log_n, q, p, dnum, psi)))


def ckks_strerror(code):
    return _lib.ckks_strerror(code).decode()


def ckks_last_error():
    return _lib.ckks_last_error().decode()


class Context:
    """Owns a ckks_ctx (device tables and workspace) for one parameter set."""

    def __init__(self, log_n, q, p, dnum, device=0, psi=None):
        self.log_n, self.q, self.p, self.dnum = int(log_n), [int(v) for v in q], [int(v) for v in p], int(dnum)
        self.N = 1 << self.log_n
        self.L, self.K = len(self.q), len(self.p)
        self.device = int(device)
        self.key_words = self.dnum * 2 * (self.L + self.K) * self.N  # one switch key [dnum][2][L+K][N]
        handle = ctypes.c_void_p()
        st = _params_struct(self.log_n, self.q, self.p, self.dnum, psi)
        _check(_lib.ckks_ctx_create(ctypes.byref(st), int(device), ctypes.byref(handle)), "ckks_ctx_create")
        self.handle = handle
        out = (ctypes.c_uint64 * (self.L + self.K))()
        _check(_lib.ckks_ctx_psi(self.handle, out), "ckks_ctx_psi")
        self.psi = [int(v) for v in out]

    def close(self):
        if self.handle:
            _check(_lib.ckks_ctx_destroy(self.handle), "ckks_ctx_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _lvl(ctx, level):
    """level + 1 when level is valid for ctx, else None (the library reports the range error)."""
    return level + 1 if 0 <= level < ctx.L else None


def _w(*factors):
    """Product of word counts, or None when any factor is None or negative."""
    r = 1
    for f in factors:
        if f is None or f < 0:
            return None
        r *= f
    return r


def ckks_ntt(ctx, data, npoly, limb_begin, n_limb, inverse, stream=None):
    _check(_lib.ckks_ntt(ctx.handle, _dev(ctx, data, _w(npoly, n_limb, ctx.N), "data"), npoly, limb_begin, n_limb,
                         int(inverse), _stream(stream)), "ckks_ntt")


def ckks_automorph(ctx, d_in, d_out, npoly, level, galois_elt, domain, stream=None):
    n = _w(npoly, _lvl(ctx, level), ctx.N)
    _check(_lib.ckks_automorph(ctx.handle, _dev(ctx, d_in, n, "d_in"), _dev(ctx, d_out, n, "d_out"), npoly, level,
                               int(galois_elt), int(domain), _stream(stream)), "ckks_automorph")


def ckks_keyswitch(ctx, d_poly, d_evk, d_out, level, stream=None):
    nl = _lvl(ctx, level)
    _check(_lib.ckks_keyswitch(ctx.handle, _dev(ctx, d_poly, _w(nl, ctx.N), "d_poly"),
                               _dev(ctx, d_evk, ctx.key_words, "d_evk"), _dev(ctx, d_out, _w(2, nl, ctx.N), "d_out"),
                               level, _stream(stream)), "ckks_keyswitch")


def _key_list(ctx, keys, galois_elts, what):
    """Host array of key pointers; a key may be None only for Galois element 1."""
    arr = (ctypes.c_void_p * max(1, len(keys)))()
    for k, (t, g) in enumerate(zip(keys, galois_elts)):
        p = _dev(ctx, t, ctx.key_words, "%s[%d]" % (what, k), optional=(int(g) == 1))
        arr[k] = p.value if p is not None else None
    return arr


def _u32_list(vals):
    return (ctypes.c_uint32 * max(1, len(vals)))(*[int(v) for v in vals])


def ckks_rotate(ctx, d_ct_in, d_ct_out, batch, level, galois_elts, d_evks, flags=0, stream=None):
    _count(galois_elts, batch, "galois_elts")
    _count(d_evks, batch, "d_evks")
    n = _w(batch, 2, _lvl(ctx, level), ctx.N)
    _check(_lib.ckks_rotate(ctx.handle, _dev(ctx, d_ct_in, n, "d_ct_in"), _dev(ctx, d_ct_out, n, "d_ct_out"), batch,
                            level, _u32_list(galois_elts), _key_list(ctx, d_evks, galois_elts, "d_evks"), flags,
                            _stream(stream)), "ckks_rotate")


def ckks_rotate_noalloc(ctx, d_ct_in, d_ct_out, batch, level, galois_elts, d_evks, flags=0, stream=None):
    """ckks_rotate with the library's fixed scratch: no allocation, everything on `stream`."""
    _count(galois_elts, batch, "galois_elts")
    _count(d_evks, batch, "d_evks")
    n = _w(batch, 2, _lvl(ctx, level), ctx.N)
    _check(_lib.ckks_rotate_noalloc(ctx.handle, _dev(ctx, d_ct_in, n, "d_ct_in"), _dev(ctx, d_ct_out, n, "d_ct_out"),
                                    batch, level, _u32_list(galois_elts),
                                    _key_list(ctx, d_evks, galois_elts, "d_evks"), flags, _stream(stream)),
           "ckks_rotate_noalloc")


def ckks_rotate_hoisted(ctx, d_ct_in, n_in, level, galois_elts, d_evks, d_ct_out, stream=None):
    n_rot = len(galois_elts)
    _count(d_evks, n_rot, "d_evks")
    ct = _w(2, _lvl(ctx, level), ctx.N)
    _check(_lib.ckks_rotate_hoisted(ctx.handle, _dev(ctx, d_ct_in, _w(n_in, ct), "d_ct_in"), n_in, level, n_rot,
                                    _u32_list(galois_elts), _key_list(ctx, d_evks, galois_elts, "d_evks"),
                                    _dev(ctx, d_ct_out, _w(n_in, n_rot, ct), "d_ct_out"), _stream(stream)),
           "ckks_rotate_hoisted")


def ckks_rescale(ctx, d_in, d_out, batch, level, stream=None):
    nl = _lvl(ctx, level)
    _check(_lib.ckks_rescale(ctx.handle, _dev(ctx, d_in, _w(batch, 2, nl, ctx.N), "d_in"),
                             _dev(ctx, d_out, _w(batch, 2, nl and nl - 1, ctx.N), "d_out"), batch, level,
                             _stream(stream)), "ckks_rescale")


def ckks_mul_relin_rescale(ctx, d_a, d_b, d_rlk, d_out, batch, level, flags=0, stream=None):
    nl = _lvl(ctx, level)
    n_in = _w(batch, 2, nl, ctx.N)
    n_out = _w(batch, 2, nl if flags & CKKS_NO_RESCALE else (nl and nl - 1), ctx.N)
    _check(_lib.ckks_mul_relin_rescale(ctx.handle, _dev(ctx, d_a, n_in, "d_a"), _dev(ctx, d_b, n_in, "d_b"),
                                       _dev(ctx, d_rlk, ctx.key_words, "d_rlk"), _dev(ctx, d_out, n_out, "d_out"),
                                       batch, level, flags, _stream(stream)), "ckks_mul_relin_rescale")


def ckks_poly_eval(ctx, d_ct_in, batch, level, scale, coeffs, d_rlk, d_ct_out, stream=None):
    """Horner evaluation of sum_k coeffs[k] x^k; returns the output scale."""
    c = (ctypes.c_double * len(coeffs))(*[float(v) for v in coeffs])
    degree = len(coeffs) - 1
    nl = _lvl(ctx, level)
    n_out = _w(batch, 2, nl and nl - degree, ctx.N) if 1 <= degree else None
    out_scale = ctypes.c_double(0.0)
    _check(_lib.ckks_poly_eval(ctx.handle, _dev(ctx, d_ct_in, _w(batch, 2, nl, ctx.N), "d_ct_in"), batch, level,
                               float(scale), c, degree, _dev(ctx, d_rlk, ctx.key_words, "d_rlk"),
                               _dev(ctx, d_ct_out, n_out, "d_ct_out"), ctypes.byref(out_scale), _stream(stream)),
           "ckks_poly_eval")
    return out_scale.value


def tree_depth(degree):
    """Levels ckks_poly_eval_tree consumes: ceil(log2(degree + 1))."""
    return degree.bit_length()


def ckks_poly_eval_tree(ctx, d_ct_in, batch, level, scale, coeffs, d_rlk, d_ct_out, stream=None):
    """Depth-efficient evaluation of sum_k coeffs[k] x^k (depth
    ceil(log2(d + 1))); returns the output scale (= scale)."""
    c = (ctypes.c_double * len(coeffs))(*[float(v) for v in coeffs])
    degree = len(coeffs) - 1
    nl = _lvl(ctx, level)
    n_out = None
    if nl is not None and 1 <= degree <= 64 and nl > tree_depth(degree):
        n_out = _w(batch, 2, nl - tree_depth(degree), ctx.N)
    out_scale = ctypes.c_double(0.0)
    _check(_lib.ckks_poly_eval_tree(ctx.handle, _dev(ctx, d_ct_in, _w(batch, 2, nl, ctx.N), "d_ct_in"), batch, level,
                                    float(scale), c, degree, _dev(ctx, d_rlk, ctx.key_words, "d_rlk"),
                                    _dev(ctx, d_ct_out, n_out, "d_ct_out"), ctypes.byref(out_scale),
                                    _stream(stream)), "ckks_poly_eval_tree")
    return out_scale.value


def _matvec_args(ctx, d_x, n_in, n_out, n1, n2, baby_galois, d_evk_baby, giant_galois, d_evk_giant, d_y, level,
                 flags, diag_words):
    _count(baby_galois, max(n1 - 1, 0), "baby_galois")
    _count(d_evk_baby, max(n1 - 1, 0), "d_evk_baby")
    _count(giant_galois, max(n2 - 1, 0), "giant_galois")
    _count(d_evk_giant, max(n2 - 1, 0), "d_evk_giant")
    nl = _lvl(ctx, level)
    pos = n_in >= 1 and n_out >= 1 and n1 >= 1 and n2 >= 1
    x = _dev(ctx, d_x, _w(n_in, 2, nl, ctx.N) if pos else None, "d_x")
    y_limbs = nl if flags & CKKS_NO_RESCALE else (nl and nl - 1)
    y = _dev(ctx, d_y, _w(n_out, 2, y_limbs, ctx.N) if pos else None, "d_y")
    gb, gg = _u32_list(baby_galois), _u32_list(giant_galois)
    kb = _key_list(ctx, d_evk_baby, [0] * len(d_evk_baby), "d_evk_baby")
    kg = _key_list(ctx, d_evk_giant, [0] * len(d_evk_giant), "d_evk_giant")
    dw = _w(n_out, n_in, n2, n1, diag_words, nl, ctx.N) if pos else None
    return x, y, gb, kb, gg, kg, dw


def ckks_ptmatvec(ctx, d_x, n_in, d_diags, n_out, n1, n2, baby_galois, d_evk_baby, giant_galois, d_evk_giant, d_y,
                  level, flags=0, stream=None):
    x, y, gb, kb, gg, kg, dw = _matvec_args(ctx, d_x, n_in, n_out, n1, n2, baby_galois, d_evk_baby, giant_galois,
                                            d_evk_giant, d_y, level, flags, 1)
    _check(_lib.ckks_ptmatvec(ctx.handle, x, n_in, _dev(ctx, d_diags, dw, "d_diags"), n_out, n1, n2, gb, kb, gg, kg,
                              y, level, flags, _stream(stream)), "ckks_ptmatvec")


def ckks_ctmatvec(ctx, d_x, n_in, d_diags, n_out, n1, n2, d_rlk, baby_galois, d_evk_baby, giant_galois, d_evk_giant,
                  d_y, level, flags=0, stream=None):
    x, y, gb, kb, gg, kg, dw = _matvec_args(ctx, d_x, n_in, n_out, n1, n2, baby_galois, d_evk_baby, giant_galois,
                                            d_evk_giant, d_y, level, flags, 2)
    _check(_lib.ckks_ctmatvec(ctx.handle, x, n_in, _dev(ctx, d_diags, dw, "d_diags"), n_out, n1, n2,
                              _dev(ctx, d_rlk, ctx.key_words, "d_rlk"), gb, kb, gg, kg, y, level, flags,
                              _stream(stream)), "ckks_ctmatvec")


def ckks_trace_begin(ctx, kernel):
    _check(_lib.ckks_trace_begin(ctx.handle, kernel.encode() if kernel else None), "ckks_trace_begin")


def ckks_trace_end(ctx):
    st = ckks_trace_stats()
    _check(_lib.ckks_trace_end(ctx.handle, ctypes.byref(st)), "ckks_trace_end")
    return {"launches": st.launches, "total_ms": st.total_ms, "work_units": st.work_units}


class KernelTrace:
    """Times every launch of one kernel family with HIP events (see ckks_trace_begin)."""

    def __init__(self, ctx, kernel):
        self.ctx, self.kernel = ctx, kernel
        ckks_trace_begin(ctx, kernel)

    def read(self):
        st = ckks_trace_end(self.ctx)
        st.update(name=self.kernel, alg_units=st["work_units"], unit_name="modmul-class ops")
        return st

    def close(self):
        pass


def ckks_probe_list():
    """Names of the device calibration probes (include/ckks_probe.h)."""
    buf = ctypes.create_string_buffer(1024)
    _check(_lib.ckks_probe_list(buf, len(buf)), "ckks_probe_list")
    return buf.value.decode().split(",")


def ckks_probe_rate(what, device=0, copy_bytes=0):
    """(rate, median ms) of one calibration probe: lane-operations per second,
    or bytes read + written per second for "copy"."""
    rate, ms = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(_lib.ckks_probe_rate(int(device), what.encode(), int(copy_bytes), ctypes.byref(rate), ctypes.byref(ms)),
           "ckks_probe_rate")
    return rate.value, ms.value
