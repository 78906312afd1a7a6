"""ctypes binding of libbdssm.so (the C ABI in include/bdssm.h).

Argument marshalling only: every step of the computation runs in the HIP kernels. The
functions take torch CUDA tensors (PyTorch provides device memory and streams), pass
their device pointers to the library, and raise ``BdssmError`` on a non-OK status.
There is no fallback: if the library is not built, loading raises.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbdssm.so")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = range(9)
STATIC_SCRATCH_BYTES = 64 << 20
F32, BF16 = 0, 1

# every symbol include/bdssm.h declares
EXPORTS = ("bdssm_abi_version", "bdssm_status_str", "bdssm_prefix_scan_workspace",
           "bdssm_prefix_scan", "bdssm_block_step", "bdssm_block_step_ex", "bdssm_commit",
           "bdssm_decode_graph_create",
           "bdssm_decode_graph_launch", "bdssm_decode_graph_destroy",
           "bdssm_conv_workspace", "bdssm_conv", "bdssm_block_step_conv", "bdssm_commit_conv",
           "bdssm_state_ops_bytes", "bdssm_state_ops", "bdssm_block_step_ops",
           "bdssm_set_launch_override", "bdssm_prefix_scan_static",
           "bdssm_full_window_workspace", "bdssm_full_window",
           "bdssm_state_bf16_bytes", "bdssm_state_bf16", "bdssm_block_step_variant",
           "bdssm_commit_refresh")
STATE_F32, STATE_OPS, STATE_BF16 = 0, 1, 2


class BdssmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("nheads", ctypes.c_int32),
                ("headdim", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("ngroups", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("y_dtype", ctypes.c_int32)]


class SeqPtrs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("dt", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("C", ctypes.c_void_p)]


class LaunchOverride(ctypes.Structure):
    _fields_ = [("block_kernel", ctypes.c_int32), ("lat_waves", ctypes.c_int32),
                ("bw_heads", ctypes.c_int32), ("bw_splits", ctypes.c_int32)]


class StepParams(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("D", ctypes.c_void_p), ("A_rev", ctypes.c_void_p),
                ("D_rev", ctypes.c_void_p), ("skip_per_channel", ctypes.c_int32)]


class ConvParams(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


_lib = None


def load():
    """Load the built library (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is not built; run bidirectional_mamba_state_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        V, P, I32, I64, SZ = ctypes.c_void_p, ctypes.POINTER, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.bdssm_abi_version.restype = ctypes.c_int
        lib.bdssm_abi_version.argtypes = []
        lib.bdssm_status_str.restype = ctypes.c_char_p
        lib.bdssm_status_str.argtypes = [ctypes.c_int]
        lib.bdssm_prefix_scan_workspace.restype = SZ
        lib.bdssm_prefix_scan_workspace.argtypes = [P(Dims), I64, I32, I32, I32]
        lib.bdssm_prefix_scan.restype = ctypes.c_int
        lib.bdssm_prefix_scan.argtypes = [P(Dims), I64, I32, P(SeqPtrs), V, V, V, V, V, V, V, SZ, V]
        lib.bdssm_block_step.restype = ctypes.c_int
        lib.bdssm_block_step.argtypes = [P(Dims), I32, V, P(SeqPtrs), P(SeqPtrs), V, V, V, V]
        lib.bdssm_block_step_ex.restype = ctypes.c_int
        lib.bdssm_block_step_ex.argtypes = [P(Dims), I32, V, P(SeqPtrs), P(SeqPtrs), V, V, V, V, V, V]
        lib.bdssm_commit.restype = ctypes.c_int
        lib.bdssm_commit.argtypes = [P(Dims), I32, P(SeqPtrs), V, V, V, V, V]
        lib.bdssm_decode_graph_create.restype = ctypes.c_int
        lib.bdssm_state_ops_bytes.restype = SZ
        lib.bdssm_state_ops_bytes.argtypes = [P(Dims)]
        lib.bdssm_state_ops.restype = ctypes.c_int
        lib.bdssm_state_ops.argtypes = [P(Dims), V, V, V]
        lib.bdssm_block_step_ops.restype = ctypes.c_int
        lib.bdssm_block_step_ops.argtypes = [P(Dims), I32, V, P(SeqPtrs), P(SeqPtrs), V, V, V, V, V, V]
        lib.bdssm_decode_graph_create.argtypes = [P(Dims), I32, I32, V, V, P(SeqPtrs), P(SeqPtrs), V, V,
                                                  P(V), P(SeqPtrs), V, V, P(V)]
        lib.bdssm_decode_graph_launch.restype = ctypes.c_int
        lib.bdssm_decode_graph_launch.argtypes = [V, V]
        lib.bdssm_decode_graph_destroy.restype = None
        lib.bdssm_decode_graph_destroy.argtypes = [V]
        lib.bdssm_conv_workspace.restype = SZ
        lib.bdssm_conv_workspace.argtypes = [P(Dims), I64]
        lib.bdssm_conv.restype = ctypes.c_int
        lib.bdssm_conv.argtypes = [P(Dims), I64, P(ConvParams), I32, V, P(SeqPtrs), P(SeqPtrs), V, V]
        lib.bdssm_block_step_conv.restype = ctypes.c_int
        lib.bdssm_block_step_conv.argtypes = [P(Dims), I32, P(ConvParams), P(ConvParams), V, V,
                                              P(SeqPtrs), P(SeqPtrs), V, V, V, V, V, V, SZ, V]
        lib.bdssm_commit_conv.restype = ctypes.c_int
        lib.bdssm_commit_conv.argtypes = [P(Dims), I32, P(ConvParams), P(SeqPtrs), V, V, V, V, V,
                                          V, SZ, V]
        lib.bdssm_prefix_scan_static.restype = ctypes.c_int
        lib.bdssm_prefix_scan_static.argtypes = [P(Dims), I64, I32, P(SeqPtrs), V, V, V, V, V, V, V]
        lib.bdssm_full_window_workspace.restype = SZ
        lib.bdssm_full_window_workspace.argtypes = [P(Dims), I64, I32]
        lib.bdssm_full_window.restype = ctypes.c_int
        lib.bdssm_full_window.argtypes = [P(Dims), I64, I32, P(SeqPtrs), P(SeqPtrs), V, V, V, V, V, V, SZ, V]
        lib.bdssm_state_bf16_bytes.restype = SZ
        lib.bdssm_state_bf16_bytes.argtypes = [P(Dims)]
        lib.bdssm_state_bf16.restype = ctypes.c_int
        lib.bdssm_state_bf16.argtypes = [P(Dims), V, V, V]
        lib.bdssm_block_step_variant.restype = ctypes.c_int
        lib.bdssm_block_step_variant.argtypes = [P(Dims), I32, V, I32, P(SeqPtrs), P(SeqPtrs), P(StepParams), V, V]
        lib.bdssm_commit_refresh.restype = ctypes.c_int
        lib.bdssm_commit_refresh.argtypes = [P(Dims), I32, P(SeqPtrs), V, V, V, V, I32, V, V]
        lib.bdssm_set_launch_override.restype = ctypes.c_int
        lib.bdssm_set_launch_override.argtypes = [P(LaunchOverride)]
        _lib = lib
    return _lib


def status_str(status):
    return load().bdssm_status_str(status).decode()


def abi_version():
    return load().bdssm_abi_version()


def _check(rc):
    if rc != OK:
        raise BdssmError(rc, status_str(rc))


def _ptr(t):
    """Device pointer of a torch CUDA tensor (None -> NULL). Refuses host tensors and
    non-contiguous views: the library takes contiguous device buffers only."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise TypeError("bdssm takes device (CUDA/HIP) tensors only")
    if not t.is_contiguous():
        raise ValueError("bdssm takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dims(batch, nheads, headdim, d_state, ngroups, in_dtype, y_dtype=F32):
    return Dims(batch, nheads, headdim, d_state, ngroups, in_dtype, y_dtype)


def _seq(s):
    if s is None:
        return None
    x, dt, B, C = s
    return SeqPtrs(_ptr(x), _ptr(dt), _ptr(B), _ptr(C))


def _byref(v):
    return None if v is None else ctypes.byref(v)


def prefix_scan_workspace(d, length, chunk, with_y, with_chunk_states):
    return load().bdssm_prefix_scan_workspace(ctypes.byref(d), length, chunk, int(with_y),
                                              int(with_chunk_states))


def prefix_scan(d, length, chunk, seq, A, D, h_init, y, chunk_states, h_out,
                workspace=None, workspace_bytes=None, stream=None):
    """bdssm_prefix_scan. seq = (x, dt, B, C) tensors; C may be None when y is None."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().bdssm_prefix_scan(ctypes.byref(d), length, chunk, _byref(_seq(seq)), _ptr(A),
                                    _ptr(D), _ptr(h_init), _ptr(y), _ptr(chunk_states),
                                    _ptr(h_out), _ptr(workspace), workspace_bytes,
                                    _stream(stream)))


def prefix_scan_static(d, length, chunk, seq, A, D, h_init, y, chunk_states, h_out, stream=None):
    """bdssm_prefix_scan_static: bdssm_prefix_scan with its workspace taken from the
    library's static scratch buffer (no workspace argument, nothing allocated)."""
    _check(load().bdssm_prefix_scan_static(ctypes.byref(d), length, chunk, _byref(_seq(seq)), _ptr(A),
                                           _ptr(D), _ptr(h_init), _ptr(y), _ptr(chunk_states),
                                           _ptr(h_out), _stream(stream)))


def full_window_workspace(d, length, chunk):
    return load().bdssm_full_window_workspace(ctypes.byref(d), length, chunk)


def full_window(d, length, chunk, fwd, rev, A, D, A_rev, D_rev, y, workspace=None, stream=None):
    """bdssm_full_window: forward and reverse scans over the whole window from zero states
    (A_rev None = A; D_rev None = no reverse skip term)."""
    _check(load().bdssm_full_window(ctypes.byref(d), length, chunk, _byref(_seq(fwd)), _byref(_seq(rev)),
                                    _ptr(A), _ptr(D), _ptr(A if A_rev is None else A_rev), _ptr(D_rev),
                                    _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def block_step(d, block_len, h_prefix, fwd, rev, A, D, y, stream=None):
    """bdssm_block_step. fwd, rev = (x, dt, B, C) tensors."""
    _check(load().bdssm_block_step(ctypes.byref(d), block_len, _ptr(h_prefix), _byref(_seq(fwd)),
                                   _byref(_seq(rev)), _ptr(A), _ptr(D), _ptr(y), _stream(stream)))


def block_step_ex(d, block_len, h_prefix, fwd, rev, A, D, A_rev, D_rev, y, stream=None):
    """bdssm_block_step_ex: separate reverse-direction decay A_rev and skip weight D_rev
    (None = no reverse skip term)."""
    _check(load().bdssm_block_step_ex(ctypes.byref(d), block_len, _ptr(h_prefix), _byref(_seq(fwd)),
                                      _byref(_seq(rev)), _ptr(A), _ptr(D), _ptr(A_rev), _ptr(D_rev),
                                      _ptr(y), _stream(stream)))


def state_ops_bytes(d):
    """bdssm_state_ops_bytes (SIZE_MAX for invalid or unsupported dims)."""
    return load().bdssm_state_ops_bytes(ctypes.byref(d))


def state_ops(d, h, ops, stream=None):
    """bdssm_state_ops: the cached state h in operand form, into ops."""
    _check(load().bdssm_state_ops(ctypes.byref(d), _ptr(h), _ptr(ops), _stream(stream)))


def block_step_ops(d, block_len, h_ops, fwd, rev, A, D, y, A_rev=None, D_rev=None, stream=None):
    """bdssm_block_step_ops: block step from the state in operand form (A_rev None = A)."""
    _check(load().bdssm_block_step_ops(ctypes.byref(d), block_len, _ptr(h_ops), _byref(_seq(fwd)),
                                       _byref(_seq(rev)), _ptr(A), _ptr(D),
                                       _ptr(A if A_rev is None else A_rev), _ptr(D_rev), _ptr(y),
                                       _stream(stream)))


KERNEL_AUTO, KERNEL_SMALL_BATCH, KERNEL_BANDWIDTH = 0, 1, 2


def set_launch_override(block_kernel=0, lat_waves=0, bw_heads=0, bw_splits=0):
    """bdssm_set_launch_override (tests and launch-shape sweeps only): pins the block-step
    kernel and its launch shape for later calls; all zeros = automatic."""
    o = LaunchOverride(block_kernel, lat_waves, bw_heads, bw_splits)
    _check(load().bdssm_set_launch_override(ctypes.byref(o)))


def state_bf16_bytes(d):
    """bdssm_state_bf16_bytes (SIZE_MAX for invalid or unsupported dims)."""
    return load().bdssm_state_bf16_bytes(ctypes.byref(d))


def state_bf16(d, h, out, stream=None):
    """bdssm_state_bf16: the bf16 copy of the cached state h, into out."""
    _check(load().bdssm_state_bf16(ctypes.byref(d), _ptr(h), _ptr(out), _stream(stream)))


def block_step_variant(d, block_len, state, state_form, fwd, rev, A, D, y, A_rev=None, D_rev=None,
                       skip_per_channel=False, stream=None):
    """bdssm_block_step_variant: the state as float32, operand form or bf16 (state_form), skip
    weights per head or per channel."""
    prm = StepParams(_ptr(A), _ptr(D), _ptr(A_rev), _ptr(D_rev), int(skip_per_channel))
    _check(load().bdssm_block_step_variant(ctypes.byref(d), block_len, _ptr(state), state_form, _byref(_seq(fwd)),
                                           _byref(_seq(rev)), ctypes.byref(prm), _ptr(y), _stream(stream)))


def commit(d, block_len, clean, A, D, h, y=None, stream=None):
    """bdssm_commit. clean = (x, dt, B, C) tensors (C may be None when y is None)."""
    _check(load().bdssm_commit(ctypes.byref(d), block_len, _byref(_seq(clean)), _ptr(A), _ptr(D),
                               _ptr(h), _ptr(y), _stream(stream)))


def commit_refresh(d, block_len, clean, A, D, h, state_copy, state_form=STATE_OPS, y=None, stream=None):
    """bdssm_commit_refresh: the commit, with the block step's copy of the advanced state
    (operand form or bf16) written in the same pass."""
    _check(load().bdssm_commit_refresh(ctypes.byref(d), block_len, _byref(_seq(clean)), _ptr(A), _ptr(D), _ptr(h),
                                       _ptr(state_copy), state_form, _ptr(y), _stream(stream)))


def conv_params(weight, bias, activation, width=None):
    """A bdssm_conv_params for weight [CH, W] and bias [CH] (or None) device tensors."""
    w = int(weight.shape[1]) if width is None else width
    return ConvParams(w, activation, _ptr(weight), _ptr(bias))


def conv_workspace(d, length):
    return load().bdssm_conv_workspace(ctypes.byref(d), length)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def conv(d, length, params, reverse, state_in, raw, out, state_out, stream=None):
    """bdssm_conv. raw, out = (x, dt, B, C) tensors (dt unused, may be None)."""
    _check(load().bdssm_conv(ctypes.byref(d), length, ctypes.byref(params), int(reverse), _ptr(state_in),
                             _byref(_seq(raw)), _byref(_seq(out)), _ptr(state_out), _stream(stream)))


def block_step_conv(d, block_len, conv_fwd, conv_rev, h_prefix, conv_state, fwd, rev, A, D, y,
                    workspace, A_rev=None, D_rev=None, stream=None):
    """bdssm_block_step_conv: fwd, rev are raw (unconvolved) inputs."""
    _check(load().bdssm_block_step_conv(ctypes.byref(d), block_len, ctypes.byref(conv_fwd),
                                        ctypes.byref(conv_rev), _ptr(h_prefix), _ptr(conv_state),
                                        _byref(_seq(fwd)), _byref(_seq(rev)), _ptr(A), _ptr(D),
                                        _ptr(A_rev), _ptr(D_rev), _ptr(y), _ptr(workspace),
                                        _nbytes(workspace), _stream(stream)))


def commit_conv(d, block_len, params, clean, A, D, h, conv_state, workspace, y=None, stream=None):
    """bdssm_commit_conv: advances h and the conv state in place over raw clean inputs."""
    _check(load().bdssm_commit_conv(ctypes.byref(d), block_len, ctypes.byref(params), _byref(_seq(clean)),
                                    _ptr(A), _ptr(D), _ptr(h), _ptr(conv_state), _ptr(y), _ptr(workspace),
                                    _nbytes(workspace), _stream(stream)))


class DecodeGraph:
    """bdssm_decode_graph_*: the steps of one active block and its commit, recorded once
    and replayed with launch(). Keeps references to the tensors whose addresses it holds."""

    def __init__(self, d, block_len, h, fwd_steps, rev_steps, A, D, ys, clean=None, y_commit=None,
                 h_ops=None):
        import torch
        steps = len(ys)
        if len(fwd_steps) != steps or len(rev_steps) != steps:
            raise ValueError("one fwd, rev and y per step")
        self._keep = (h, h_ops, fwd_steps, rev_steps, A, D, ys, clean, y_commit)
        fw = (SeqPtrs * max(steps, 1))(*[_seq(s) for s in fwd_steps])
        rv = (SeqPtrs * max(steps, 1))(*[_seq(s) for s in rev_steps])
        yp = (ctypes.c_void_p * max(steps, 1))(*[_ptr(t) for t in ys])
        # record on a side stream: the legacy default stream cannot be captured
        side = torch.cuda.Stream()
        handle = ctypes.c_void_p()
        rc = load().bdssm_decode_graph_create(ctypes.byref(d), block_len, steps, _ptr(h), _ptr(h_ops), fw, rv,
                                              _ptr(A), _ptr(D), yp, _byref(_seq(clean)),
                                              _ptr(y_commit), side.cuda_stream, ctypes.byref(handle))
        _check(rc)
        self._handle = handle

    def launch(self, stream=None):
        _check(load().bdssm_decode_graph_launch(self._handle, _stream(stream)))

    def close(self):
        if getattr(self, "_handle", None):
            load().bdssm_decode_graph_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ data movement helpers
def to_device(arr, device="cuda"):
    """numpy input array (float32, or uint16 bfloat16 patterns) -> torch device tensor."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def seq_to_device(seq, device="cuda"):
    """An inputs.Seq -> (x, dt, B, C) device tensors."""
    return tuple(to_device(a, device) for a in (seq.x, seq.dt, seq.B, seq.C))
