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
    "ckks_ntt", "ckks_automorph", "ckks_keyswitch", "ckks_rotate", "ckks_rotate_hoisted", "ckks_rescale",
    "ckks_mul_relin_rescale", "ckks_poly_eval", "ckks_ptmatvec", "ckks_ctmatvec", "ckks_trace_begin",
    "ckks_trace_end",
]

# Kernel whose launches take the largest share of a rotation batch (by
# rocprofv3 time): the forward row pass fused with the key inner product.
DOMINANT_KERNEL = "ntt_row_ip"
# int32 VALU operations per 64-bit modmul-class operation: the 10 32x32-bit
# partial products of a 64-bit Shoup (or Barrett) multiplication plus 6 int32
# adds/subtracts to combine them and apply the quotient.
OPS_PER_MODMUL = 16


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
        "ckks_rotate_hoisted": (i, [vp, vp, i, i, i, u32p, pp, vp, vp]),
        "ckks_rescale": (i, [vp, vp, vp, i, i, vp]),
        "ckks_mul_relin_rescale": (i, [vp, vp, vp, vp, vp, i, i, ctypes.c_uint, vp]),
        "ckks_poly_eval": (i, [vp, vp, i, i, ctypes.c_double, ctypes.POINTER(ctypes.c_double), i, vp, vp,
                               ctypes.POINTER(ctypes.c_double), vp]),
        "ckks_ptmatvec": (i, [vp, vp, i, vp, i, i, i, u32p, pp, u32p, pp, vp, i, ctypes.c_uint, vp]),
        "ckks_ctmatvec": (i, [vp, vp, i, vp, i, i, i, vp, u32p, pp, u32p, pp, vp, i, ctypes.c_uint, vp]),
        "ckks_trace_begin": (i, [vp, ctypes.c_char_p]),
        "ckks_trace_end": (i, [vp, ctypes.POINTER(ckks_trace_stats)]),
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


def _ptr(t):
    """Device pointer of a contiguous int64 torch tensor (or None)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if t.element_size() != 8:
        raise ValueError("tensor must hold 64-bit words")
    return ctypes.c_void_p(t.data_ptr())


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


def ckks_ntt(ctx, data, npoly, limb_begin, n_limb, inverse, stream=None):
    _check(_lib.ckks_ntt(ctx.handle, _ptr(data), npoly, limb_begin, n_limb, int(inverse), _stream(stream)),
           "ckks_ntt")


def ckks_automorph(ctx, d_in, d_out, npoly, level, galois_elt, domain, stream=None):
    _check(_lib.ckks_automorph(ctx.handle, _ptr(d_in), _ptr(d_out), npoly, level, int(galois_elt), int(domain),
                               _stream(stream)), "ckks_automorph")


def ckks_keyswitch(ctx, d_poly, d_evk, d_out, level, stream=None):
    _check(_lib.ckks_keyswitch(ctx.handle, _ptr(d_poly), _ptr(d_evk), _ptr(d_out), level, _stream(stream)),
           "ckks_keyswitch")


def _ptr_list(tensors):
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for k, t in enumerate(tensors):
        arr[k] = t.data_ptr() if t is not None else None
    return arr


def ckks_rotate(ctx, d_ct_in, d_ct_out, batch, level, galois_elts, d_evks, flags=0, stream=None):
    g = (ctypes.c_uint32 * max(1, batch))(*[int(v) for v in galois_elts])
    _check(_lib.ckks_rotate(ctx.handle, _ptr(d_ct_in), _ptr(d_ct_out), batch, level, g, _ptr_list(d_evks),
                            flags, _stream(stream)), "ckks_rotate")


def ckks_rotate_hoisted(ctx, d_ct_in, n_in, level, galois_elts, d_evks, d_ct_out, stream=None):
    n_rot = len(galois_elts)
    g = (ctypes.c_uint32 * max(1, n_rot))(*[int(v) for v in galois_elts])
    _check(_lib.ckks_rotate_hoisted(ctx.handle, _ptr(d_ct_in), n_in, level, n_rot, g, _ptr_list(d_evks),
                                    _ptr(d_ct_out), _stream(stream)), "ckks_rotate_hoisted")


def ckks_rescale(ctx, d_in, d_out, batch, level, stream=None):
    _check(_lib.ckks_rescale(ctx.handle, _ptr(d_in), _ptr(d_out), batch, level, _stream(stream)), "ckks_rescale")


def ckks_mul_relin_rescale(ctx, d_a, d_b, d_rlk, d_out, batch, level, flags=0, stream=None):
    _check(_lib.ckks_mul_relin_rescale(ctx.handle, _ptr(d_a), _ptr(d_b), _ptr(d_rlk), _ptr(d_out), batch, level,
                                       flags, _stream(stream)), "ckks_mul_relin_rescale")


def ckks_poly_eval(ctx, d_ct_in, batch, level, scale, coeffs, d_rlk, d_ct_out, stream=None):
    """Horner evaluation of sum_k coeffs[k] x^k; returns the output scale."""
    c = (ctypes.c_double * len(coeffs))(*[float(v) for v in coeffs])
    out_scale = ctypes.c_double(0.0)
    _check(_lib.ckks_poly_eval(ctx.handle, _ptr(d_ct_in), batch, level, float(scale), c, len(coeffs) - 1,
                               _ptr(d_rlk), _ptr(d_ct_out), ctypes.byref(out_scale), _stream(stream)),
           "ckks_poly_eval")
    return out_scale.value


def ckks_ptmatvec(ctx, d_x, n_in, d_diags, n_out, n1, n2, baby_galois, d_evk_baby, giant_galois, d_evk_giant, d_y,
                  level, flags=0, stream=None):
    gb = (ctypes.c_uint32 * max(1, n1 - 1))(*[int(v) for v in baby_galois])
    gg = (ctypes.c_uint32 * max(1, n2 - 1))(*[int(v) for v in giant_galois])
    _check(_lib.ckks_ptmatvec(ctx.handle, _ptr(d_x), n_in, _ptr(d_diags), n_out, n1, n2, gb, _ptr_list(d_evk_baby),
                              gg, _ptr_list(d_evk_giant), _ptr(d_y), level, flags, _stream(stream)),
           "ckks_ptmatvec")


def ckks_ctmatvec(ctx, d_x, n_in, d_diags, n_out, n1, n2, d_rlk, baby_galois, d_evk_baby, giant_galois, d_evk_giant,
                  d_y, level, flags=0, stream=None):
    gb = (ctypes.c_uint32 * max(1, n1 - 1))(*[int(v) for v in baby_galois])
    gg = (ctypes.c_uint32 * max(1, n2 - 1))(*[int(v) for v in giant_galois])
    _check(_lib.ckks_ctmatvec(ctx.handle, _ptr(d_x), n_in, _ptr(d_diags), n_out, n1, n2, _ptr(d_rlk), gb,
                              _ptr_list(d_evk_baby), gg, _ptr_list(d_evk_giant), _ptr(d_y), level, flags,
                              _stream(stream)),
           "ckks_ctmatvec")


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
        st.update(name=self.kernel, alg_units=st["work_units"], ops_per_unit=OPS_PER_MODMUL,
                  unit_name="modmul-class ops")
        return st

    def close(self):
        pass
