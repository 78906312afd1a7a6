"""Python access to the CPU float64 oracle (``bdssm_oracle.c``).

TEST INFRASTRUCTURE ONLY: the oracle is the plain sequential recurrence that the HIP
path is checked against. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it. It does not import the HIP package, and
the HIP package never imports it.

Arrays come in as numpy: inputs are float32 or uint16 bfloat16 bit patterns (decoded
exactly by the C code), states and outputs are float64.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bdssm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force=True):
    """Compile the oracle with gcc (plain -O2, OpenMP over independent heads)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("nheads", ctypes.c_int32),
                ("headdim", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("in_dtype", ctypes.c_int32)]


class _Seq(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dt", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("C", ctypes.c_void_p)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_scan.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, ctypes.c_int64,
                                    ctypes.POINTER(_Seq), P, P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_block_step.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, P,
                                          ctypes.POINTER(_Seq), ctypes.POINTER(_Seq),
                                          P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_block_step_ex.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, P,
                                             ctypes.POINTER(_Seq), ctypes.POINTER(_Seq),
                                             P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_block_step_dch.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, P,
                                              ctypes.POINTER(_Seq), ctypes.POINTER(_Seq),
                                              P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_full_window.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, ctypes.POINTER(_Seq),
                                           ctypes.POINTER(_Seq), P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_commit.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64,
                                      ctypes.POINTER(_Seq), P, P, P, P, P, ctypes.c_int]
        lib.oracle_conv.argtypes = [ctypes.POINTER(_Dims), ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, P, P, P,
                                    ctypes.POINTER(_Seq), ctypes.POINTER(_Seq), P, ctypes.c_int]
        for f in (lib.oracle_scan, lib.oracle_block_step, lib.oracle_block_step_ex, lib.oracle_commit,
                  lib.oracle_conv, lib.oracle_full_window, lib.oracle_block_step_dch):
            f.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads():
    return _load().oracle_max_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data


def _in(a, dtype):
    want = np.uint16 if dtype == 1 else np.float32
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"oracle input must be {np.dtype(want)}, got {a.dtype}")
    return a


class _Call:
    """Holds the contiguous arrays alive for the duration of one C call."""

    def __init__(self, seq):
        self.dtype = seq.dtype
        self.x, self.dt, self.B, self.C = (_in(a, seq.dtype) for a in (seq.x, seq.dt, seq.B, seq.C))
        self.s = _Seq(_ptr(self.x), _ptr(self.dt), _ptr(self.B), _ptr(self.C))


def _dims(seq, ngroups):
    b, _, H, P = seq.x.shape
    N = seq.B.shape[3]
    return _Dims(b, H, P, N, ngroups, seq.dtype)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _mask(heads, H):
    if heads is None:
        return None
    m = np.zeros(H, dtype=np.int8)
    m[list(heads)] = 1
    return m


def scan(seq, A, D, chunk, h_init=None, want_y=True, want_chunk_states=True, heads=None,
         nthreads=0):
    """Prefix scan. Returns (y [b,len,H,P] or None, chunk_states [b,nch,H,N,P] or None,
    h_out [b,H,N,P]); all float64. ``heads``: optional subset of heads to compute."""
    c = _Call(seq)
    b, L, H, P = seq.x.shape
    G, N = seq.B.shape[2], seq.B.shape[3]
    nch = -(-L // chunk)
    y = np.zeros((b, L, H, P)) if want_y else None
    cs = np.zeros((b, nch, H, N, P)) if want_chunk_states else None
    h_out = np.zeros((b, H, N, P))
    hi = _f64(h_init)
    A = np.ascontiguousarray(A, np.float32)
    D = np.ascontiguousarray(D, np.float32)
    m = _mask(heads, H)
    rc = _load().oracle_scan(ctypes.byref(_dims(seq, G)), L, chunk, ctypes.byref(c.s),
                             _ptr(A), _ptr(D), _ptr(hi), _ptr(y), _ptr(cs), _ptr(h_out),
                             _ptr(m), nthreads)
    if rc:
        raise ValueError("oracle_scan rejected its arguments")
    return y, cs, h_out


def block_step(h_prefix, fwd, rev, A, D, heads=None, nthreads=0, A_rev=None, D_rev=None):
    """Block step. Returns (y, y_fwd, y_rev), each [b,T,H,P] float64; y includes D x_fwd.
    With A_rev and/or D_rev (separate reverse-direction parameters, oracle_block_step_ex)
    the reverse scan decays with A_rev and y also includes D_rev x_rev."""
    cf, cr = _Call(fwd), _Call(rev)
    b, T, H, P = fwd.x.shape
    G = fwd.B.shape[2]
    y = np.zeros((b, T, H, P))
    yf = np.zeros_like(y)
    yr = np.zeros_like(y)
    hp = _f64(h_prefix)
    A = np.ascontiguousarray(A, np.float32)
    D = np.ascontiguousarray(D, np.float32)
    m = _mask(heads, H)
    if A_rev is None and D_rev is None:
        rc = _load().oracle_block_step(ctypes.byref(_dims(fwd, G)), T, _ptr(hp), ctypes.byref(cf.s),
                                       ctypes.byref(cr.s), _ptr(A), _ptr(D), _ptr(y), _ptr(yf),
                                       _ptr(yr), _ptr(m), nthreads)
    else:
        Ar = None if A_rev is None else np.ascontiguousarray(A_rev, np.float32)
        Dr = None if D_rev is None else np.ascontiguousarray(D_rev, np.float32)
        rc = _load().oracle_block_step_ex(ctypes.byref(_dims(fwd, G)), T, _ptr(hp), ctypes.byref(cf.s),
                                          ctypes.byref(cr.s), _ptr(A), _ptr(D), _ptr(Ar), _ptr(Dr),
                                          _ptr(y), _ptr(yf), _ptr(yr), _ptr(m), nthreads)
    if rc:
        raise ValueError("oracle_block_step rejected its arguments")
    return y, yf, yr


def block_step_per_channel(h_prefix, fwd, rev, A, D, A_rev=None, D_rev=None, heads=None, nthreads=0):
    """Block step with skip weights per head and channel (oracle_block_step_dch): D and D_rev
    (optional) are [H, P]. Returns y [b, T, H, P] float64."""
    cf, cr = _Call(fwd), _Call(rev)
    b, T, H, P = fwd.x.shape
    G = fwd.B.shape[2]
    y = np.zeros((b, T, H, P))
    hp = _f64(h_prefix)
    A = np.ascontiguousarray(A, np.float32)
    D = np.ascontiguousarray(D, np.float32)
    assert D.shape == (H, P)
    Ar = None if A_rev is None else np.ascontiguousarray(A_rev, np.float32)
    Dr = None if D_rev is None else np.ascontiguousarray(D_rev, np.float32)
    assert Dr is None or Dr.shape == (H, P)
    m = _mask(heads, H)
    rc = _load().oracle_block_step_dch(ctypes.byref(_dims(fwd, G)), T, _ptr(hp), ctypes.byref(cf.s),
                                       ctypes.byref(cr.s), _ptr(A), _ptr(D), _ptr(Ar), _ptr(Dr), _ptr(y),
                                       _ptr(m), nthreads)
    if rc:
        raise ValueError("oracle_block_step_dch rejected its arguments")
    return y


def full_window(fwd, rev, A, D, A_rev=None, D_rev=None, heads=None, nthreads=0):
    """Full-window bidirectional scan (oracle_full_window): forward from zero over the whole
    window of fwd, reverse from zero at its end over rev (decay A_rev, default A), plus
    D x_fwd (and D_rev x_rev). Returns y [b, len, H, P] float64."""
    cf, cr = _Call(fwd), _Call(rev)
    b, L, H, P = fwd.x.shape
    G = fwd.B.shape[2]
    y = np.zeros((b, L, H, P))
    A = np.ascontiguousarray(A, np.float32)
    D = np.ascontiguousarray(D, np.float32)
    Ar = None if A_rev is None else np.ascontiguousarray(A_rev, np.float32)
    Dr = None if D_rev is None else np.ascontiguousarray(D_rev, np.float32)
    m = _mask(heads, H)
    rc = _load().oracle_full_window(ctypes.byref(_dims(fwd, G)), L, ctypes.byref(cf.s), ctypes.byref(cr.s),
                                    _ptr(A), _ptr(D), _ptr(Ar), _ptr(Dr), _ptr(y), _ptr(m), nthreads)
    if rc:
        raise ValueError("oracle_full_window rejected its arguments")
    return y


def commit(h, clean, A, D, want_y=False, heads=None, nthreads=0):
    """Commit. Returns (h_new [b,H,N,P], y [b,T,H,P] or None), float64; h is not modified."""
    c = _Call(clean)
    b, T, H, P = clean.x.shape
    G = clean.B.shape[2]
    hn = np.array(h, dtype=np.float64, copy=True, order="C")
    y = np.zeros((b, T, H, P)) if want_y else None
    A = np.ascontiguousarray(A, np.float32)
    D = np.ascontiguousarray(D, np.float32)
    m = _mask(heads, H)
    rc = _load().oracle_commit(ctypes.byref(_dims(clean, G)), T, ctypes.byref(c.s), _ptr(A),
                               _ptr(D), _ptr(hn), _ptr(y), _ptr(m), nthreads)
    if rc:
        raise ValueError("oracle_commit rejected its arguments")
    return hn, y


class ConvSeq:
    """A token segment produced by ``conv``: x, dt, B, C arrays of the input dtype."""

    def __init__(self, x, dt, B, C, dtype):
        self.x, self.dt, self.B, self.C, self.dtype = x, dt, B, C, dtype

    @property
    def length(self):
        return self.x.shape[1]


def conv_channels(seq):
    b, _, H, P = seq.x.shape
    G, N = seq.B.shape[2], seq.B.shape[3]
    return H * P + 2 * G * N


def conv(seq, weight, bias, act, reverse=False, state_in=None, want_state=True, nthreads=0):
    """Depthwise convolution + activation of the x, B, C channels (oracle_conv).

    weight [CH, W] float32 (CH = H*P + 2*G*N, channels x, B, C), bias [CH] float32 or None,
    act 0 (identity) or 1 (SiLU), state_in [b, W-1, CH] in the input dtype or None (zero
    history). Returns (out, state_out): out has the input's dt and the convolved x, B, C
    rounded to the input dtype; state_out [b, W-1, CH] (forward only, else None)."""
    c = _Call(seq)
    b, L, H, P = seq.x.shape
    G = seq.B.shape[2]
    CH = conv_channels(seq)
    weight = np.ascontiguousarray(weight, np.float32)
    W = weight.shape[1]
    assert weight.shape == (CH, W)
    bias = None if bias is None else np.ascontiguousarray(bias, np.float32)
    dt_np = np.uint16 if seq.dtype == 1 else np.float32
    out = ConvSeq(np.zeros_like(c.x), c.dt, np.zeros_like(c.B), np.zeros_like(c.C), seq.dtype)
    o = _Seq(_ptr(out.x), _ptr(out.dt), _ptr(out.B), _ptr(out.C))
    si = None if state_in is None else _in(state_in, seq.dtype)
    so = np.zeros((b, W - 1, CH), dtype=dt_np) if (want_state and not reverse) else None
    rc = _load().oracle_conv(ctypes.byref(_dims(seq, G)), L, W, act, 1 if reverse else 0,
                             _ptr(weight), _ptr(bias), _ptr(si), ctypes.byref(c.s), ctypes.byref(o),
                             _ptr(so), nthreads)
    if rc:
        raise ValueError("oracle_conv rejected its arguments")
    return out, so


def block_step_conv(h_prefix, conv_state, fwd, rev, conv_fwd, conv_rev, A, D, heads=None,
                    nthreads=0, A_rev=None, D_rev=None):
    """Block step on raw (pre-convolution) inputs: the forward branch's x, B, C are
    convolved causally from the cached conv state, the reverse branch's anti-causally inside
    the block, then the block step of eqs. (11)-(13). conv_fwd / conv_rev: (weight, bias,
    act). Returns (y, y_fwd, y_rev)."""
    pf, _ = conv(fwd, *conv_fwd, reverse=False, state_in=conv_state, want_state=False, nthreads=nthreads)
    pr, _ = conv(rev, *conv_rev, reverse=True, nthreads=nthreads)
    return block_step(h_prefix, pf, pr, A, D, heads=heads, nthreads=nthreads, A_rev=A_rev, D_rev=D_rev)


def commit_conv(h, conv_state, clean, conv_fwd, A, D, want_y=False, heads=None, nthreads=0):
    """Commit on raw inputs: convolve the clean block from the conv state, advance the SSM
    state over it, and advance the conv state. Returns (h_new, conv_state_new, y or None)."""
    pc, so = conv(clean, *conv_fwd, reverse=False, state_in=conv_state, nthreads=nthreads)
    hn, y = commit(h, pc, A, D, want_y=want_y, heads=heads, nthreads=nthreads)
    return hn, so, y
