"""The C ABI on the CPU: the library loads, exports every symbol include/bdssm.h declares,
and rejects bad arguments before launching anything. No call here reaches a kernel:
every argument set is one the validation refuses."""
import ctypes
import os
import re

import pytest

from bidirectional_mamba_state_amd import bdssm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    text = open(os.path.join(ROOT, "include", "bdssm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bdssm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(bdssm.LIB_PATH)
    syms = header_symbols()
    assert syms == sorted(bdssm.EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s
    assert bdssm.abi_version() == 4
    for st in range(9):
        assert bdssm.status_str(st).startswith("BDSSM_")
    assert "unknown" in bdssm.status_str(99)


FAKE = 0x100000  # 16-byte aligned, never dereferenced (every call below is rejected first)


def seq(x=FAKE, dt=FAKE, B=FAKE, C=FAKE):
    return bdssm.SeqPtrs(x, dt, B, C)


def call_prefix(d, length=64, chunk=64, s=None, A=FAKE, D=FAKE, h_init=None, y=None, cs=None,
                h_out=FAKE + 4096, ws=None, wsb=0):
    lib = bdssm.load()
    s = seq() if s is None else s
    return lib.bdssm_prefix_scan(None if d is None else ctypes.byref(d), length, chunk,
                                 ctypes.byref(s), A, D, h_init, y, cs, h_out, ws, wsb, None)


def call_block(d, T=16, h=FAKE, f=None, r=None, A=FAKE, D=FAKE, y=FAKE + (1 << 24)):
    lib = bdssm.load()
    f = seq() if f is None else f
    r = seq() if r is None else r
    return lib.bdssm_block_step(None if d is None else ctypes.byref(d), T, h, ctypes.byref(f),
                                ctypes.byref(r), A, D, y, None)


def call_commit(d, T=16, c=None, A=FAKE, D=FAKE, h=FAKE + (1 << 24), y=None):
    lib = bdssm.load()
    c = seq() if c is None else c
    return lib.bdssm_commit(None if d is None else ctypes.byref(d), T, ctypes.byref(c), A, D, h, y, None)


def good():
    return bdssm.dims(1, 4, 16, 16, 1, bdssm.F32, bdssm.F32)


def test_null_dims_and_pointers():
    assert call_prefix(None) == bdssm.ERR_NULL
    assert call_block(None) == bdssm.ERR_NULL
    assert call_commit(None) == bdssm.ERR_NULL
    assert call_prefix(good(), h_out=None) == bdssm.ERR_NULL
    assert call_prefix(good(), s=seq(x=None)) == bdssm.ERR_NULL
    assert call_prefix(good(), s=seq(C=None), y=FAKE + (1 << 26)) == bdssm.ERR_NULL  # C needed for y
    assert call_block(good(), h=None) == bdssm.ERR_NULL
    assert call_block(good(), r=seq(B=None)) == bdssm.ERR_NULL
    assert call_block(good(), y=None) == bdssm.ERR_NULL
    assert call_commit(good(), h=None) == bdssm.ERR_NULL
    assert call_commit(good(), c=seq(C=None), y=FAKE + (1 << 26)) == bdssm.ERR_NULL


def test_shapes_and_unsupported():
    d = good()
    d.ngroups = 3
    assert call_prefix(d) == bdssm.ERR_SHAPE           # H % G != 0
    d = good()
    d.nheads = 0
    assert call_block(d) == bdssm.ERR_SHAPE
    d = good()
    d.batch = -1
    assert call_commit(d) == bdssm.ERR_SHAPE
    assert call_prefix(good(), length=-1) == bdssm.ERR_SHAPE
    assert call_block(good(), T=-1) == bdssm.ERR_SHAPE
    assert call_commit(good(), T=-1) == bdssm.ERR_SHAPE
    assert call_block(good(), T=257) == bdssm.ERR_UNSUPPORTED
    assert call_prefix(good(), chunk=48) == bdssm.ERR_UNSUPPORTED
    d = good()
    d.d_state = 32                                      # no kernel for (32, 16)
    assert call_prefix(d) == bdssm.ERR_UNSUPPORTED
    d = good()
    d.in_dtype = 7
    assert call_block(d) == bdssm.ERR_UNSUPPORTED
    assert bdssm.prefix_scan_workspace(d, 64, 64, True, True) == ctypes.c_size_t(-1).value


def test_alignment_and_alias():
    assert call_prefix(good(), s=seq(x=FAKE + 2)) == bdssm.ERR_ALIGN
    assert call_block(good(), h=FAKE + 8) == bdssm.ERR_ALIGN
    assert call_commit(good(), A=FAKE + 4) == bdssm.ERR_ALIGN
    # y on top of x
    assert call_block(good(), y=FAKE) == bdssm.ERR_ALIAS
    assert call_prefix(good(), y=FAKE, cs=None) == bdssm.ERR_ALIAS
    # h_out partially overlapping h_init (exact aliasing is allowed)
    assert call_prefix(good(), h_init=FAKE + (1 << 24), h_out=FAKE + (1 << 24) + 16) == bdssm.ERR_ALIAS
    # commit state on top of the clean inputs
    assert call_commit(good(), h=FAKE) == bdssm.ERR_ALIAS


def test_workspace_query_and_missing_workspace():
    # fp32 inputs (vector-ALU path): chunk-local states are kept for the y pass, in
    # chunk_states when given, else in the workspace
    d32 = bdssm.dims(1, 48, 64, 128, 1, bdssm.F32, bdssm.F32)
    assert bdssm.prefix_scan_workspace(d32, 8192, 256, True, False) >= 32 * 48 * 128 * 64 * 4
    assert bdssm.prefix_scan_workspace(d32, 8192, 256, True, True) < 1 << 20
    assert bdssm.prefix_scan_workspace(d32, 0, 256, True, True) == 0
    # bf16 inputs (matrix-core path): 48 (stream, head) pairs are too few to fill the GPU,
    # so the tokens are split into segments whose entering states live in the workspace
    d = bdssm.dims(1, 48, 64, 128, 1, bdssm.BF16, bdssm.F32)
    need = bdssm.prefix_scan_workspace(d, 8192, 256, True, False)
    assert need >= 2 * 48 * 128 * 64 * 4
    assert bdssm.prefix_scan_workspace(d, 8192, 256, True, True) == need
    assert bdssm.prefix_scan_workspace(d, 0, 256, True, True) == 0
    base = 1 << 32
    s = seq(base, base + (1 << 28), base + (2 << 28), base + (3 << 28))
    rc = call_prefix(d, length=8192, chunk=256, s=s, A=base + (4 << 28), D=base + (5 << 28),
                     y=base + (6 << 28), h_out=base + (7 << 28), ws=None, wsb=0)
    assert rc == bdssm.ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    d = good()
    with pytest.raises(TypeError):
        bdssm.block_step(d, 16, torch.zeros(4), None, None, None, None, None, stream=0)


def test_decode_graph_argument_checks():
    """bdssm_decode_graph_*: argument errors are reported before any HIP call."""
    lib = bdssm.load()
    d = good()
    out = ctypes.c_void_p(1234)
    f = (bdssm.SeqPtrs * 2)(seq(), seq())
    ys = (ctypes.c_void_p * 2)(FAKE + (1 << 24), FAKE + (1 << 25))
    create = lib.bdssm_decode_graph_create
    # NULL stream (the legacy default stream cannot be captured); out is cleared
    assert create(ctypes.byref(d), 16, 2, FAKE, None, f, f, FAKE, FAKE, ys, None, None, None,
                  ctypes.byref(out)) == bdssm.ERR_NULL
    assert out.value is None
    assert create(None, 16, 2, FAKE, None, f, f, FAKE, FAKE, ys, None, None, FAKE, ctypes.byref(out)) == bdssm.ERR_NULL
    assert create(ctypes.byref(d), 16, 2, FAKE, None, f, f, FAKE, FAKE, ys, None, None, FAKE, None) == bdssm.ERR_NULL
    assert create(ctypes.byref(d), 16, -1, FAKE, None, f, f, FAKE, FAKE, ys, None, None, FAKE,
                  ctypes.byref(out)) == bdssm.ERR_SHAPE
    assert create(ctypes.byref(d), 16, 2, FAKE, None, None, f, FAKE, FAKE, ys, None, None, FAKE,
                  ctypes.byref(out)) == bdssm.ERR_NULL
    # no steps and no commit: nothing to record
    assert create(ctypes.byref(d), 16, 0, FAKE, None, None, None, FAKE, FAKE, None, None, None, FAKE,
                  ctypes.byref(out)) == bdssm.ERR_NULL
    assert lib.bdssm_decode_graph_launch(None, None) == bdssm.ERR_NULL
    lib.bdssm_decode_graph_destroy(None)


def test_block_step_ex_argument_checks():
    lib = bdssm.load()
    d = good()
    f, r = seq(), seq()

    def call(A_rev=FAKE + 64, D_rev=None, y=FAKE + (1 << 24)):
        return lib.bdssm_block_step_ex(ctypes.byref(d), 16, FAKE, ctypes.byref(f), ctypes.byref(r),
                                       FAKE, FAKE, A_rev, D_rev, y, None)
    assert call(A_rev=None) == bdssm.ERR_NULL          # the reverse decay is required
    assert call(A_rev=FAKE + 4) == bdssm.ERR_ALIGN
    assert call(D_rev=FAKE + 8) == bdssm.ERR_ALIGN
    assert call(A_rev=FAKE + (1 << 24)) == bdssm.ERR_ALIAS   # y on top of A_rev
    assert call(D_rev=FAKE + (1 << 24)) == bdssm.ERR_ALIAS   # y on top of D_rev


def test_conv_argument_checks():
    """bdssm_conv, bdssm_block_step_conv, bdssm_commit_conv: argument errors are reported
    before anything is launched; the workspace query's size."""
    lib = bdssm.load()
    d = bdssm.dims(1, 4, 16, 16, 1, bdssm.BF16, bdssm.F32)   # CH = 64 + 32 = 96
    # one convolved copy of 10 tokens: x 1280 B, B and C 320 B each, 256-byte aligned parts
    assert bdssm.conv_workspace(d, 10) == 1280 + 512 + 512
    assert bdssm.conv_workspace(d, -1) == ctypes.c_size_t(-1).value
    base = 1 << 32
    raw = seq(base, None, base + (1 << 20), base + (2 << 20))
    out = seq(base + (3 << 20), None, base + (4 << 20), base + (5 << 20))
    W = base + (6 << 20)
    st = base + (7 << 20)

    def conv(cp=None, reverse=0, si=st, so=st, r=raw, o=out, length=10):
        cp = bdssm.ConvParams(4, 1, W, None) if cp is None else cp
        return lib.bdssm_conv(ctypes.byref(d), length, ctypes.byref(cp), reverse, si, ctypes.byref(r),
                              ctypes.byref(o), so, None)
    assert lib.bdssm_conv(ctypes.byref(d), 10, None, 0, None, ctypes.byref(raw), ctypes.byref(out), None,
                          None) == bdssm.ERR_NULL
    assert conv(bdssm.ConvParams(5, 1, W, None)) == bdssm.ERR_UNSUPPORTED
    assert conv(bdssm.ConvParams(0, 1, W, None)) == bdssm.ERR_UNSUPPORTED
    assert conv(bdssm.ConvParams(4, 2, W, None)) == bdssm.ERR_UNSUPPORTED
    assert conv(bdssm.ConvParams(4, 1, None, None)) == bdssm.ERR_NULL
    assert conv(bdssm.ConvParams(4, 1, W + 4, None)) == bdssm.ERR_ALIGN
    assert conv(reverse=1) == bdssm.ERR_SHAPE               # no state for the reverse branch
    assert conv(length=-1) == bdssm.ERR_SHAPE
    assert conv(si=st + 8) == bdssm.ERR_ALIGN
    assert conv(so=st + 16) == bdssm.ERR_ALIAS               # partial overlap of the two states
    assert conv(o=seq(base + 64, None, base + (4 << 20), base + (5 << 20))) == bdssm.ERR_ALIAS  # out on raw
    assert conv(o=seq(base + (3 << 20), None, None, base + (5 << 20))) == bdssm.ERR_NULL
    assert conv(so=W) == bdssm.ERR_ALIAS                     # state on the weights
    # block step with conv
    f = seq(base, base + (8 << 20), base + (1 << 20), base + (2 << 20))
    r = seq(base + (9 << 20), base + (10 << 20), base + (11 << 20), base + (12 << 20))
    cp = bdssm.ConvParams(4, 1, W, None)
    ws = base + (16 << 20)
    need = 2 * bdssm.conv_workspace(d, 10)

    def step(cs=st, wsp=ws, wsb=need, y=base + (20 << 20)):
        return lib.bdssm_block_step_conv(ctypes.byref(d), 10, ctypes.byref(cp), ctypes.byref(cp),
                                         base + (24 << 20), cs, ctypes.byref(f), ctypes.byref(r), FAKE,
                                         FAKE + 256, None, None, y, wsp, wsb, None)
    assert step(cs=None) == bdssm.ERR_NULL                   # width 4 needs the conv state
    assert step(wsb=need - 1) == bdssm.ERR_WORKSPACE
    assert step(wsp=None) == bdssm.ERR_WORKSPACE
    assert step(wsp=base + (1 << 20)) == bdssm.ERR_ALIAS     # workspace on an input
    assert step(y=ws) == bdssm.ERR_ALIAS                      # y on the workspace
    assert step(y=base + (1 << 20)) == bdssm.ERR_ALIAS       # y on a raw input
    # commit with conv: C is required (it enters the conv state)
    cl = seq(base, base + (8 << 20), base + (1 << 20), None)
    assert lib.bdssm_commit_conv(ctypes.byref(d), 10, ctypes.byref(cp), ctypes.byref(cl), FAKE, FAKE + 256,
                                 base + (24 << 20), st, None, ws, need, None) == bdssm.ERR_NULL
    cl = seq(base, base + (8 << 20), base + (1 << 20), base + (2 << 20))
    assert lib.bdssm_commit_conv(ctypes.byref(d), 10, ctypes.byref(cp), ctypes.byref(cl), FAKE, FAKE + 256,
                                 base + (24 << 20), st, None, ws, 16, None) == bdssm.ERR_WORKSPACE
    assert lib.bdssm_commit_conv(ctypes.byref(d), 10, ctypes.byref(cp), ctypes.byref(cl), FAKE, FAKE + 256,
                                 base + (24 << 20), base + 32, None, ws, need, None) == bdssm.ERR_ALIAS


def test_state_ops_argument_checks():
    """bdssm_state_ops_bytes, bdssm_state_ops, bdssm_block_step_ops: sizes, and argument
    errors reported before anything is launched."""
    lib = bdssm.load()
    d = bdssm.dims(2, 4, 64, 128, 1, bdssm.BF16, bdssm.F32)
    nbytes = 2 * 4 * 128 * 64 * 4
    assert bdssm.state_ops_bytes(d) == nbytes
    assert bdssm.state_ops_bytes(good()) == ctypes.c_size_t(-1).value      # (16, 16): unsupported
    assert bdssm.state_ops_bytes(bdssm.dims(1, 4, 64, 128, 3, bdssm.BF16)) == ctypes.c_size_t(-1).value
    h, ops = FAKE, FAKE + (1 << 24)
    st = lib.bdssm_state_ops
    assert st(ctypes.byref(d), None, ops, None) == bdssm.ERR_NULL
    assert st(ctypes.byref(d), h, None, None) == bdssm.ERR_NULL
    assert st(ctypes.byref(good()), h, ops, None) == bdssm.ERR_UNSUPPORTED
    assert st(ctypes.byref(d), h + 8, ops, None) == bdssm.ERR_ALIGN
    assert st(ctypes.byref(d), h, h + nbytes - 16, None) == bdssm.ERR_ALIAS
    f, r = seq(), seq()

    def step(dd=d, T=32, h_ops=ops, y=FAKE + (1 << 26), A_rev=FAKE):
        return lib.bdssm_block_step_ops(ctypes.byref(dd), T, h_ops, ctypes.byref(f), ctypes.byref(r),
                                        FAKE, FAKE, A_rev, None, y, None)
    assert step(h_ops=None) == bdssm.ERR_NULL
    assert step(A_rev=None) == bdssm.ERR_NULL
    assert step(y=ops + 1024) == bdssm.ERR_ALIAS                       # y on top of the state
    assert step(T=129) == bdssm.ERR_UNSUPPORTED                        # longer than the kernels' blocks
    assert step(dd=bdssm.dims(2, 4, 64, 128, 1, bdssm.F32)) == bdssm.ERR_UNSUPPORTED   # fp32 inputs
    assert step(T=-1) == bdssm.ERR_SHAPE
    assert step(T=0) == bdssm.OK                                       # nothing to do


def test_missing_library_raises(monkeypatch):
    # no fallback path: without the built library every call raises
    monkeypatch.setattr(bdssm, "_lib", None)
    monkeypatch.setattr(bdssm, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libbdssm.so"))
    with pytest.raises(OSError, match="not built"):
        bdssm.abi_version()
    with pytest.raises(OSError, match="not built"):
        bdssm.load()


def test_launch_override_validation():
    """bdssm_set_launch_override accepts the documented values only, and NULL resets."""
    lib = bdssm.load()
    bad = [(3, 0, 0, 0), (-1, 0, 0, 0), (0, 3, 0, 0), (0, 1, 0, 0), (0, 0, -2, 0), (0, 0, 0, 3)]
    for v in bad:
        o = bdssm.LaunchOverride(*v)
        assert lib.bdssm_set_launch_override(ctypes.byref(o)) == bdssm.ERR_UNSUPPORTED, v
    for v in [(1, 2, 0, 0), (2, 4, 6, 2), (0, 0, 0, 4)]:
        o = bdssm.LaunchOverride(*v)
        assert lib.bdssm_set_launch_override(ctypes.byref(o)) == bdssm.OK, v
    assert lib.bdssm_set_launch_override(None) == bdssm.OK
    bdssm.set_launch_override()
    with pytest.raises(bdssm.BdssmError):
        bdssm.set_launch_override(lat_waves=5)


def test_prefix_scan_static_rejects_oversized_plans():
    """bdssm_prefix_scan_static refuses, before any launch, a call whose plan needs more
    workspace than the static scratch buffer holds (float32 inputs: the chunk-local states
    of every chunk live in the workspace, 1 KiB each at d_state = headdim = 16)."""
    lib = bdssm.load()
    d = bdssm.dims(1, 64, 16, 16, 1, bdssm.F32, bdssm.F32)
    L, chunk = 1 << 20, 16
    need = bdssm.prefix_scan_workspace(d, L, chunk, True, False)
    assert need > bdssm.STATIC_SCRATCH_BYTES
    x, y = 1 << 40, 1 << 42   # far apart: no range overlaps, nothing dereferenced
    s = bdssm.SeqPtrs(x, x + (1 << 38), x + (2 << 38), x + (3 << 38))
    rc = lib.bdssm_prefix_scan_static(ctypes.byref(d), L, chunk, ctypes.byref(s), FAKE, FAKE + 4096, None,
                                      y, None, FAKE + 8192, None)
    assert rc == bdssm.ERR_SCRATCH
    assert "static scratch" in bdssm.status_str(rc)
    # the usual validation comes first
    assert lib.bdssm_prefix_scan_static(None, L, chunk, ctypes.byref(s), FAKE, FAKE, None, y, None,
                                        FAKE + 8192, None) == bdssm.ERR_NULL


def test_full_window_validation():
    """bdssm_full_window validates before any launch: NULL pointers, shapes, chunks, aliasing
    of y with the inputs, and the workspace (the prefix scan's with outputs)."""
    lib = bdssm.load()
    d = bdssm.dims(1, 4, 64, 128, 1, bdssm.BF16, bdssm.F32)
    L = 4096
    need = lib.bdssm_full_window_workspace(ctypes.byref(d), L, 256)
    assert need == bdssm.prefix_scan_workspace(d, L, 256, True, False) and need > 0
    base = 1 << 40
    f = bdssm.SeqPtrs(base, base + (1 << 36), base + (2 << 36), base + (3 << 36))
    r = bdssm.SeqPtrs(base + (4 << 36), base + (5 << 36), base + (6 << 36), base + (7 << 36))
    y = base + (8 << 36)
    ws = base + (9 << 36)

    def call(dd=d, length=L, chunk=256, fw=f, rv=r, A=FAKE, D=FAKE + 256, Ar=FAKE + 512, Dr=None, yy=y, w=ws,
             wb=need):
        return lib.bdssm_full_window(None if dd is None else ctypes.byref(dd), length, chunk,
                                     None if fw is None else ctypes.byref(fw), None if rv is None else ctypes.byref(rv),
                                     A, D, Ar, Dr, yy, w, wb, None)

    assert call(dd=None) == bdssm.ERR_NULL
    assert call(fw=None) == bdssm.ERR_NULL
    assert call(rv=bdssm.SeqPtrs(base, base, base, None)) == bdssm.ERR_NULL     # C is needed
    assert call(Ar=None) == bdssm.ERR_NULL
    assert call(yy=None) == bdssm.ERR_NULL
    assert call(length=-1) == bdssm.ERR_SHAPE
    assert call(chunk=48) == bdssm.ERR_UNSUPPORTED
    assert call(yy=y + 2) == bdssm.ERR_ALIGN
    assert call(yy=f.x) == bdssm.ERR_ALIAS                                     # y over an input
    assert call(w=None, wb=0) == bdssm.ERR_WORKSPACE
    assert call(wb=need - 1) == bdssm.ERR_WORKSPACE
    assert call(w=r.B) == bdssm.ERR_ALIAS                                      # workspace over an input
    assert call(length=0) == bdssm.OK                                          # nothing to do
