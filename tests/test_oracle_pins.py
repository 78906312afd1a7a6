"""Pins of the float64 oracle against facts other than itself.

The pages print no numeric example for the scan, so the oracle is pinned by:
  * a hand-worked example (tests/golden/hand_worked_n1p1.json);
  * the quadratic "state-space dual" form of the same recurrence, brute-forced in numpy
    on tiny inputs (a different formula: a sum over all source tokens with cumulative
    log-decays, instead of a token-by-token recurrence);
  * closed forms (one token; A = 0 gives a cumulative sum; constant decay gives a
    geometric series);
  * invariants: reverse == flip . forward . flip, associativity of the scan (scan of
    U||V from h0 == scan of V from the state after U), linearity, group replication;
  * planted mistakes: a copy of the oracle with one plausible error compiled on the CPU
    must fail these pins.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from bidirectional_mamba_state_amd.inputs import Seq, round_bf16_bits, bf16_bits_to_f32

HERE = os.path.dirname(os.path.abspath(__file__))
F32, BF16 = 0, 1


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


def rand_seq(rng, b, L, H, P, N, G, dtype=F32):
    x = rng.standard_normal((b, L, H, P))
    dt = np.clip(np.log1p(np.exp(rng.normal(-3.0, 1.0, (b, L, H)))), 1e-3, 0.5)
    B = 0.25 * rng.standard_normal((b, L, G, N))
    C = 0.25 * rng.standard_normal((b, L, G, N))
    if dtype == BF16:
        cv = round_bf16_bits
    else:
        def cv(v):
            return v.astype(np.float32)
    return Seq(cv(x), cv(dt), cv(B), cv(C), dtype)


def dec(seq):
    f = (lambda a: bf16_bits_to_f32(a).astype(np.float64)) if seq.dtype == BF16 else \
        (lambda a: np.asarray(a, np.float64))
    return f(seq.x), f(seq.dt), f(seq.B), f(seq.C)


def rand_params(rng, H):
    A = (-np.exp(rng.uniform(0, np.log(16), H))).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    return A, D


# ---------------------------------------------------------------- quadratic (dual) form
def quad_forward(seq, A, D, h0, with_D=True):
    """y_t = exp(cs_t) C_t.h0 + sum_{s<=t} exp(cs_t - cs_s) dt_s (C_t.B_s) x_s (+ D x_t),
    S_t = exp(cs_t) h0 + sum_{s<=t} exp(cs_t - cs_s) dt_s B_s x_s^T, with cs the
    inclusive cumulative sum of dt*A. Returns (y [b,L,H,P], states [b,L,H,N,P])."""
    x, dt, B, C = dec(seq)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros((b, L, H, P))
    S = np.zeros((b, L, H, N, P))
    tril = np.tril(np.ones((L, L)))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            cs = np.cumsum(dt[bi, :, h] * np.float64(A[h]))
            W = np.exp(np.where(tril > 0, cs[:, None] - cs[None, :], -np.inf))  # [t, s]
            Wd = W * dt[bi, None, :, h]
            CB = C[bi, :, g, :] @ B[bi, :, g, :].T
            y[bi, :, h] = (np.exp(cs)[:, None] * (C[bi, :, g, :] @ h0[bi, h])
                           + (CB * Wd) @ x[bi, :, h])
            if with_D:
                y[bi, :, h] += np.float64(D[h]) * x[bi, :, h]
            S[bi, :, h] = (np.exp(cs)[:, None, None] * h0[bi, h][None]
                           + np.einsum("ts,sn,sp->tnp", Wd, B[bi, :, g, :], x[bi, :, h]))
    return y, S


def quad_reverse(seq, A):
    """y_t = sum_{s>=t} exp(sum_{k=t}^{s-1} dt_k A) dt_s (C_t.B_s) x_s (zero state at the
    right end of the block)."""
    x, dt, B, C = dec(seq)
    b, L, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    y = np.zeros((b, L, H, P))
    triu = np.triu(np.ones((L, L)))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            a = dt[bi, :, h] * np.float64(A[h])
            rcs = np.cumsum(a[::-1])[::-1]                  # rcs_t = sum_{k>=t} a_k
            W = np.exp(np.where(triu > 0, rcs[:, None] - rcs[None, :], -np.inf))
            CB = C[bi, :, g, :] @ B[bi, :, g, :].T
            y[bi, :, h] = (CB * W * dt[bi, None, :, h]) @ x[bi, :, h]
    return y


# ------------------------------------------------------------------------- tests
def _golden_seq(d):
    a = lambda k: np.array(d[k], np.float32).reshape(1, -1, 1, 1)
    dt = np.array(d["dt"], np.float32).reshape(1, -1, 1)
    return Seq(a("x"), dt, a("B"), a("C"), F32)


def test_golden_hand_worked():
    g = json.load(open(os.path.join(HERE, "golden", "hand_worked_n1p1.json")))
    A = np.array([g["A"]], np.float32)
    D = np.array([g["D"]], np.float32)
    h0 = np.full((1, 1, 1, 1), g["h0"])
    fwd, rev = _golden_seq(g["fwd"]), _golden_seq(g["rev"])
    y, cs, hT = oracle.scan(fwd, A, D, chunk=1, h_init=h0)
    tol = 1e-6  # A = -ln2 is rounded to float32
    np.testing.assert_allclose(y.ravel(), g["scan_y_with_D"], rtol=tol, atol=tol)
    np.testing.assert_allclose(cs.ravel(), g["scan_states"], rtol=tol, atol=tol)
    np.testing.assert_allclose(hT.ravel(), g["scan_states"][-1:], rtol=tol, atol=tol)
    yb, yf, yr = oracle.block_step(h0, fwd, rev, A, D)
    np.testing.assert_allclose(yf.ravel(), g["block_y_fwd"], rtol=tol, atol=tol)
    np.testing.assert_allclose(yr.ravel(), g["block_y_rev"], rtol=tol, atol=tol)
    np.testing.assert_allclose(yb.ravel(), g["block_y"], rtol=tol, atol=tol)
    hc, yc = oracle.commit(h0, fwd, A, D, want_y=True)
    np.testing.assert_allclose(hc.ravel(), g["scan_states"][-1:], rtol=tol, atol=tol)
    np.testing.assert_allclose(yc.ravel(), g["scan_y_with_D"], rtol=tol, atol=tol)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("G", [1, 2])
def test_scan_matches_quadratic_form(dtype, G):
    rng = np.random.default_rng(11 + G + 10 * dtype)
    b, L, H, P, N, Q = 2, 40, 4, 5, 6, 16
    seq = rand_seq(rng, b, L, H, P, N, G, dtype)
    A, D = rand_params(rng, H)
    h0 = rng.standard_normal((b, H, N, P))
    y, cs, hT = oracle.scan(seq, A, D, chunk=Q, h_init=h0)
    yq, Sq = quad_forward(seq, A, D, h0)
    assert rel(y, yq) < 1e-12
    assert rel(y - np.float64(D)[None, None, :, None] * dec(seq)[0],
               yq - np.float64(D)[None, None, :, None] * dec(seq)[0]) < 1e-12
    ends = [min(L, (c + 1) * Q) - 1 for c in range(-(-L // Q))]
    assert rel(cs, Sq[:, ends]) < 1e-12          # state after each chunk (ragged tail too)
    assert rel(hT, Sq[:, -1]) < 1e-12


@pytest.mark.parametrize("G", [1, 2])
def test_block_step_matches_quadratic_form(G):
    rng = np.random.default_rng(5 + G)
    b, T, H, P, N = 2, 24, 4, 3, 5
    fwd = rand_seq(rng, b, T, H, P, N, G)
    rev = rand_seq(rng, b, T, H, P, N, G)
    A, D = rand_params(rng, H)
    h0 = rng.standard_normal((b, H, N, P))
    h0_copy = h0.copy()
    y, yf, yr = oracle.block_step(h0, fwd, rev, A, D)
    yfq, _ = quad_forward(fwd, A, D, h0, with_D=False)
    yrq = quad_reverse(rev, A)
    assert rel(yf, yfq) < 1e-12
    assert rel(yr, yrq) < 1e-12
    xf = dec(fwd)[0]
    assert rel(y, yfq + yrq + np.float64(D)[None, None, :, None] * xf) < 1e-12
    assert np.array_equal(h0, h0_copy)           # the cached state is never written


def test_block_step_separate_reverse_params():
    """Separate reverse-direction parameters: the reverse scan decays with A_rev (quadratic
    form with A_rev), y gains D_rev x_rev; with A_rev = A and no D_rev the plain step."""
    rng = np.random.default_rng(12)
    b, T, H, P, N, G = 2, 24, 4, 3, 5, 2
    fwd = rand_seq(rng, b, T, H, P, N, G)
    rev = rand_seq(rng, b, T, H, P, N, G)
    A, D = rand_params(rng, H)
    Ar, Dr = rand_params(rng, H)
    h0 = 0.3 * rng.standard_normal((b, H, N, P))
    y, yf, yr = oracle.block_step(h0, fwd, rev, A, D, A_rev=Ar, D_rev=Dr)
    qf, _ = quad_forward(fwd, A, D, h0, with_D=False)
    qr = quad_reverse(rev, Ar)
    xf, xr = dec(fwd)[0], dec(rev)[0]
    expect = qf + qr + np.float64(1) * D[None, None, :, None] * xf + Dr[None, None, :, None] * xr
    assert rel(yf, qf) < 1e-12
    assert rel(yr, qr) < 1e-12
    assert rel(y, expect) < 1e-12
    y0, _, _ = oracle.block_step(h0, fwd, rev, A, D)
    y1, _, _ = oracle.block_step(h0, fwd, rev, A, D, A_rev=A)
    assert np.array_equal(y0, y1)


def test_block_step_per_channel_skip():
    """Skip weights per head and channel: the dual form with D[h][p] x[t][p] (and
    D_rev[h][p] x_rev[t][p]); with every channel of a head equal to D[h] it is the
    per-head step exactly."""
    rng = np.random.default_rng(14)
    b, T, H, P, N, G = 2, 24, 4, 3, 5, 2
    fwd = rand_seq(rng, b, T, H, P, N, G)
    rev = rand_seq(rng, b, T, H, P, N, G)
    A, D = rand_params(rng, H)
    Ar, Dr = rand_params(rng, H)
    Dc = rng.standard_normal((H, P)).astype(np.float32)
    Drc = rng.standard_normal((H, P)).astype(np.float32)
    h0 = 0.3 * rng.standard_normal((b, H, N, P))
    y = oracle.block_step_per_channel(h0, fwd, rev, A, Dc, A_rev=Ar, D_rev=Drc)
    qf, _ = quad_forward(fwd, A, D, h0, with_D=False)
    qr = quad_reverse(rev, Ar)
    xf, xr = dec(fwd)[0], dec(rev)[0]
    assert rel(y, qf + qr + Dc[None, None] * xf + Drc[None, None] * xr) < 1e-12
    y1 = oracle.block_step_per_channel(h0, fwd, rev, A, np.repeat(D[:, None], P, 1))
    y0, _, _ = oracle.block_step(h0, fwd, rev, A, D)
    assert np.array_equal(y0, y1)


def test_reverse_is_flipped_forward():
    rng = np.random.default_rng(3)
    b, T, H, P, N, G = 1, 20, 2, 4, 3, 1
    rev = rand_seq(rng, b, T, H, P, N, G)
    zero_fwd = Seq(np.zeros_like(rev.x), rev.dt, rev.B, rev.C, rev.dtype)
    A, D = rand_params(rng, H)
    y, _, yr = oracle.block_step(np.zeros((b, H, N, P)), zero_fwd, rev, A, D)
    flip = Seq(*(np.ascontiguousarray(a[:, ::-1]) for a in (rev.x, rev.dt, rev.B, rev.C)), rev.dtype)
    yflip, _, _ = oracle.scan(flip, A, np.zeros(H, np.float32), chunk=T)
    assert rel(yr, yflip[:, ::-1]) < 1e-14
    assert rel(y, yr) < 1e-14                   # zero forward input and state: y = y_rev


@pytest.mark.parametrize("G", [1, 2])
def test_full_window_matches_quadratic_form(G):
    """The full-window bidirectional scan against the dual form over the whole window: the
    causal sum from a zero state at the start, the anti-causal sum from a zero state past the
    end (with the reverse decay), and both skip terms."""
    rng = np.random.default_rng(31 + G)
    b, L, H, P, N = 2, 37, 4, 3, 5
    fwd = rand_seq(rng, b, L, H, P, N, G)
    rev = rand_seq(rng, b, L, H, P, N, G)
    A, D = rand_params(rng, H)
    Ar, Dr = rand_params(rng, H)
    y = oracle.full_window(fwd, rev, A, D, A_rev=Ar, D_rev=Dr)
    qf, _ = quad_forward(fwd, A, D, np.zeros((b, H, N, P)), with_D=False)
    qr = quad_reverse(rev, Ar)
    xf, xr = dec(fwd)[0], dec(rev)[0]
    assert rel(y, qf + qr + D[None, None, :, None] * xf + Dr[None, None, :, None] * xr) < 1e-12
    y2 = oracle.full_window(fwd, rev, A, D)
    assert rel(y2, qf + quad_reverse(rev, A) + D[None, None, :, None] * xf) < 1e-12


def test_full_window_reverse_is_flipped_forward_scan():
    """With no forward input, the full window's output is the forward scan of the flipped
    reverse inputs, flipped back."""
    rng = np.random.default_rng(33)
    b, L, H, P, N, G = 2, 50, 3, 4, 6, 1
    rev = rand_seq(rng, b, L, H, P, N, G)
    zero_fwd = Seq(np.zeros_like(rev.x), rev.dt, rev.B, rev.C, rev.dtype)
    A, _ = rand_params(rng, H)
    y = oracle.full_window(zero_fwd, rev, A, np.zeros(H, np.float32))
    flip = Seq(*(np.ascontiguousarray(a[:, ::-1]) for a in (rev.x, rev.dt, rev.B, rev.C)), rev.dtype)
    yflip, _, _ = oracle.scan(flip, A, np.zeros(H, np.float32), chunk=16, want_chunk_states=False)
    assert rel(y, yflip[:, ::-1]) < 1e-13


def test_full_window_on_the_block_equals_the_block_step():
    """On the active block's tokens, the full-window scan over prefix || block equals the
    block step from the prefix's state: the forward scan carries the prefix in its state and
    the reverse scan reaches the block's tokens before any prefix token. On prefix tokens it
    does not equal the prefix scan's outputs: their reverse states depend on the block."""
    rng = np.random.default_rng(34)
    b, L, T, H, P, N, G = 2, 45, 13, 4, 3, 5, 2
    pre = rand_seq(rng, b, L, H, P, N, G)
    pre_rev = rand_seq(rng, b, L, H, P, N, G)
    fwd = rand_seq(rng, b, T, H, P, N, G)
    rev = rand_seq(rng, b, T, H, P, N, G)
    A, D = rand_params(rng, H)
    cat = lambda u, v: Seq(*(np.concatenate([p, q], axis=1) for p, q in zip((u.x, u.dt, u.B, u.C),
                                                                             (v.x, v.dt, v.B, v.C))), u.dtype)
    y = oracle.full_window(cat(pre, fwd), cat(pre_rev, rev), A, D)
    _, _, h = oracle.scan(pre, A, D, chunk=16, want_y=False, want_chunk_states=False)
    yb, _, _ = oracle.block_step(h, fwd, rev, A, D)
    assert rel(y[:, L:], yb) < 1e-12
    # the prefix tokens' outputs change with the block's reverse inputs
    rev2 = Seq(rev.x * np.float32(2), rev.dt, rev.B, rev.C, rev.dtype)
    y2 = oracle.full_window(cat(pre, fwd), cat(pre_rev, rev2), A, D)
    assert rel(y2[:, :L], y[:, :L]) > 1e-6


def test_scan_associativity_and_commit_chain():
    rng = np.random.default_rng(4)
    b, H, P, N, G = 2, 4, 3, 4, 2
    U = rand_seq(rng, b, 37, H, P, N, G)
    V = rand_seq(rng, b, 29, H, P, N, G)
    A, D = rand_params(rng, H)
    h0 = rng.standard_normal((b, H, N, P))
    UV = Seq(*(np.concatenate([u, v], axis=1) for u, v in
               zip((U.x, U.dt, U.B, U.C), (V.x, V.dt, V.B, V.C))), U.dtype)
    yUV, _, hUV = oracle.scan(UV, A, D, chunk=8, h_init=h0)
    _, _, hU = oracle.scan(U, A, D, chunk=8, h_init=h0)
    yV, _, hV = oracle.scan(V, A, D, chunk=8, h_init=hU)
    assert rel(hV, hUV) < 1e-13
    assert rel(yV, yUV[:, 37:]) < 1e-13
    # commits of consecutive pieces == one scan over their concatenation
    h = h0.copy()
    for s in range(0, 66, 11):
        piece = Seq(*(np.ascontiguousarray(a[:, s:s + 11]) for a in (UV.x, UV.dt, UV.B, UV.C)), UV.dtype)
        h, yc = oracle.commit(h, piece, A, D, want_y=True)
        assert rel(yc, yUV[:, s:s + 11]) < 1e-13
    assert rel(h, hUV) < 1e-13


def test_closed_forms():
    # one token: h = alpha h0 + dt B x^T, y = C.h + D x
    rng = np.random.default_rng(6)
    H, P, N = 3, 4, 5
    s1 = rand_seq(rng, 1, 1, H, P, N, 1)
    A, D = rand_params(rng, H)
    h0 = rng.standard_normal((1, H, N, P))
    y, _, hT = oracle.scan(s1, A, D, chunk=4, h_init=h0)
    x, dt, B, C = dec(s1)
    for h in range(H):
        al = np.exp(dt[0, 0, h] * np.float64(A[h]))
        hh = al * h0[0, h] + dt[0, 0, h] * np.outer(B[0, 0, 0], x[0, 0, h])
        assert rel(hT[0, h], hh) < 1e-14
        assert rel(y[0, 0, h], C[0, 0, 0] @ hh + np.float64(D[h]) * x[0, 0, h]) < 1e-14
    # A = 0: no decay, the state is the running sum of dt B x^T
    L = 30
    s = rand_seq(rng, 1, L, H, P, N, 1)
    _, cs, hT = oracle.scan(s, np.zeros(H, np.float32), D, chunk=1)
    x, dt, B, C = dec(s)
    incr = np.einsum("th,tn,thp->thnp", dt[0], B[0, :, 0], x[0])
    assert rel(cs[0], np.cumsum(incr, axis=0)) < 1e-13
    # constant dt, B, x: geometric series h_t = a^(t+1) h0 + w (1 - a^(t+1)) / (1 - a)
    dtc = np.full((1, L, H), 0.05, np.float32)
    Bc = np.tile(s.B[:, :1], (1, L, 1, 1))
    xc = np.tile(s.x[:, :1], (1, L, 1, 1))
    sc = Seq(xc, dtc, Bc, s.C, F32)
    h0 = rng.standard_normal((1, H, N, P))
    _, cs, _ = oracle.scan(sc, A, D, chunk=1, h_init=h0)
    for h in range(H):
        a = np.exp(np.float64(np.float32(0.05)) * np.float64(A[h]))
        w = np.float64(np.float32(0.05)) * np.outer(np.float64(Bc[0, 0, 0]), np.float64(xc[0, 0, h]))
        k = np.arange(1, L + 1)[:, None, None]
        ref = a ** k * h0[0, h][None] + w[None] * (1 - a ** k) / (1 - a)
        assert rel(cs[0, :, h], ref) < 1e-13


def test_linearity_and_zero():
    rng = np.random.default_rng(8)
    b, L, H, P, N, G = 1, 25, 2, 3, 4, 1
    s = rand_seq(rng, b, L, H, P, N, G)
    A, D = rand_params(rng, H)
    # dyadic inputs so that x1 + 2 x2 is exact in float32
    x1 = (np.round(rng.standard_normal(s.x.shape) * 64) / 64).astype(np.float32)
    x2 = (np.round(rng.standard_normal(s.x.shape) * 64) / 64).astype(np.float32)
    h1 = np.round(rng.standard_normal((b, H, N, P)) * 64) / 64
    h2 = np.round(rng.standard_normal((b, H, N, P)) * 64) / 64
    mk = lambda x: Seq(x, s.dt, s.B, s.C, F32)
    y1, c1, _ = oracle.scan(mk(x1), A, D, chunk=5, h_init=h1)
    y2, c2, _ = oracle.scan(mk(x2), A, D, chunk=5, h_init=h2)
    y12, c12, _ = oracle.scan(mk(x1 + 2 * x2), A, D, chunk=5, h_init=h1 + 2 * h2)
    assert rel(y12, y1 + 2 * y2) < 1e-13
    assert rel(c12, c1 + 2 * c2) < 1e-13
    # exact: zero input and zero state give exactly zero (SSM part and D part)
    y0, c0, hT0 = oracle.scan(mk(np.zeros_like(x1)), A, D, chunk=5)
    assert not y0.any() and not c0.any() and not hT0.any()


def test_group_replication():
    rng = np.random.default_rng(9)
    b, L, H, P, N = 1, 21, 4, 3, 5
    s = rand_seq(rng, b, L, H, P, N, 1)
    A, D = rand_params(rng, H)
    s2 = Seq(s.x, s.dt, np.ascontiguousarray(np.repeat(s.B, 2, axis=2)),
             np.ascontiguousarray(np.repeat(s.C, 2, axis=2)), F32)
    y1, c1, h1 = oracle.scan(s, A, D, chunk=7)
    y2, c2, h2 = oracle.scan(s2, A, D, chunk=7)
    assert np.array_equal(y1, y2) and np.array_equal(c1, c2) and np.array_equal(h1, h2)


def test_head_subset_matches_full():
    rng = np.random.default_rng(10)
    s = rand_seq(rng, 2, 17, 4, 3, 4, 2)
    A, D = rand_params(rng, 4)
    y, c, h = oracle.scan(s, A, D, chunk=8)
    ys, cs_, hs = oracle.scan(s, A, D, chunk=8, heads=[1, 3])
    assert np.array_equal(y[:, :, [1, 3]], ys[:, :, [1, 3]])
    assert np.array_equal(h[:, [1, 3]], hs[:, [1, 3]])
    assert not hs[:, [0, 2]].any()


# ------------------------------------------------------------ planted mistakes

# ---------------------------------------------------------------- convolution state
def raw_channels(seq):
    """[b, L, CH] float64 view of a segment's x, B, C channels (x, then B, then C)."""
    x, _, B, C = dec(seq)
    b, L = x.shape[:2]
    return np.concatenate([x.reshape(b, L, -1), B.reshape(b, L, -1), C.reshape(b, L, -1)], axis=2)


def conv_reference(u, w, bias, act, reverse, hist=None):
    """Depthwise convolution by shifted slices of a padded array (numpy), then the
    activation (SiLU via scipy's logistic function); float64, not rounded."""
    from scipy.special import expit
    b, L, CH = u.shape
    W = w.shape[1]
    pad = np.zeros((b, W - 1, CH)) if hist is None else hist
    ext = np.concatenate([u, pad], axis=1) if reverse else np.concatenate([pad, u], axis=1)
    out = np.zeros((b, L, CH)) + (0.0 if bias is None else bias.astype(np.float64))
    for k in range(W):
        # forward: w[k] meets u_{t-(W-1)+k}; reverse: w[k] meets u_{t+(W-1)-k}
        sl = ext[:, W - 1 - k:W - 1 - k + L] if reverse else ext[:, k:k + L]
        out = out + w[:, k].astype(np.float64) * sl
    return out * expit(out) if act == 1 else out


def rounded(v, dtype):
    return bf16_bits_to_f32(round_bf16_bits(v)).astype(np.float64) if dtype == BF16 else \
        v.astype(np.float32).astype(np.float64)


def conv_weights(rng, CH, W):
    bound = 1.0 / np.sqrt(W)
    return (rng.uniform(-bound, bound, (CH, W)).astype(np.float32),
            rng.uniform(-bound, bound, CH).astype(np.float32))


def state_f64(a, dtype):
    return bf16_bits_to_f32(a).astype(np.float64) if dtype == BF16 else np.asarray(a, np.float64)


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("reverse", [False, True])
def test_conv_matches_shifted_slices(dtype, reverse):
    """oracle_conv == the convolution written as shifted slices of a padded array, with a
    conv-state history (forward) or zeros past the block's end (reverse), SiLU, rounded
    to the input dtype; the new conv state is the extended input's last W-1 raw rows."""
    rng = np.random.default_rng(21)
    b, L, H, P, N, G, W = 2, 13, 4, 3, 5, 2, 4
    seq = rand_seq(rng, b, L, H, P, N, G, dtype)
    CH = H * P + 2 * G * N
    w, bias = conv_weights(rng, CH, W)
    hist_raw = rng.standard_normal((b, W - 1, CH))
    hist = round_bf16_bits(hist_raw) if dtype == BF16 else hist_raw.astype(np.float32)
    out, so = oracle.conv(seq, w, bias, 1, reverse=reverse, state_in=None if reverse else hist)
    u = raw_channels(seq)
    ref = conv_reference(u, w, bias, 1, reverse, None if reverse else state_f64(hist, dtype))
    got = raw_channels(out)
    want = rounded(ref, dtype)
    # the activation's exp may differ by an ulp between libm and scipy: at most one output
    # ulp apart, and almost always equal
    ulp = 2.0 ** -7 if dtype == BF16 else 2.0 ** -23
    assert np.all(np.abs(got - want) <= ulp * np.abs(want) + 1e-300)
    assert np.mean(got != want) < 1e-3
    assert np.array_equal(out.dt, seq.dt)            # dt is not convolved
    if reverse:
        assert so is None
    else:
        ext = np.concatenate([state_f64(hist, dtype), u], axis=1)
        assert np.array_equal(state_f64(so, dtype), ext[:, -(W - 1):])


def test_conv_identity_shift_and_flip():
    rng = np.random.default_rng(22)
    b, L, H, P, N, G = 1, 9, 2, 4, 3, 1
    seq = rand_seq(rng, b, L, H, P, N, G, BF16)
    CH = H * P + 2 * G * N
    # width 1, weight 1, no bias, identity: the raw input, bit for bit
    out, so = oracle.conv(seq, np.ones((CH, 1), np.float32), None, 0)
    for a, r in zip((out.x, out.B, out.C), (seq.x, seq.B, seq.C)):
        assert np.array_equal(a, r)
    assert so.shape == (b, 0, CH)
    # a unit tap on the oldest position delays by W-1 tokens, reading the conv state first
    W = 4
    w = np.zeros((CH, W), np.float32)
    w[:, 0] = 1.0
    hist = round_bf16_bits(rng.standard_normal((b, W - 1, CH)))
    out, _ = oracle.conv(seq, w, None, 0, state_in=hist)
    ext = np.concatenate([state_f64(hist, BF16), raw_channels(seq)], axis=1)
    assert np.array_equal(raw_channels(out), ext[:, :L])
    # reverse: the same tap reads W-1 tokens ahead, zero past the end
    out, _ = oracle.conv(seq, w, None, 0, reverse=True)
    u = raw_channels(seq)
    assert np.array_equal(raw_channels(out)[:, :L - 3], u[:, 3:])
    assert np.all(raw_channels(out)[:, L - 3:] == 0)
    # reverse == flip . forward from a zero history . flip
    w, bias = conv_weights(rng, CH, W)
    fl = Seq(*(np.ascontiguousarray(a[:, ::-1]) for a in (seq.x, seq.dt, seq.B, seq.C)), BF16)
    o_r, _ = oracle.conv(seq, w, bias, 1, reverse=True)
    o_f, _ = oracle.conv(fl, w, bias, 1, state_in=None)
    assert np.array_equal(raw_channels(o_r), raw_channels(o_f)[:, ::-1])


def test_conv_state_chains_and_silu_values():
    rng = np.random.default_rng(23)
    b, H, P, N, G, W = 2, 2, 4, 3, 1, 4
    U = rand_seq(rng, b, 7, H, P, N, G, BF16)
    V = rand_seq(rng, b, 2, H, P, N, G, BF16)   # shorter than the history
    X = rand_seq(rng, b, 5, H, P, N, G, BF16)
    CH = H * P + 2 * G * N
    w, bias = conv_weights(rng, CH, W)
    cat = Seq(*(np.concatenate(z, axis=1) for z in zip((U.x, U.dt, U.B, U.C), (V.x, V.dt, V.B, V.C),
                                                        (X.x, X.dt, X.B, X.C))), BF16)
    full, s_full = oracle.conv(cat, w, bias, 1)
    s = None
    outs = []
    for piece in (U, V, X):
        o, s = oracle.conv(piece, w, bias, 1, state_in=s)
        outs.append(raw_channels(o))
    assert np.array_equal(np.concatenate(outs, axis=1), raw_channels(full))
    assert np.array_equal(s, s_full)
    # SiLU closed form: width 1, unit weight, no bias
    vals = np.array([-4.0, -1.0, -0.25, 0.0, 0.5, 1.0, 3.0], np.float32)
    one = Seq(vals.reshape(1, 7, 1, 1), np.full((1, 7, 1), 0.01, np.float32),
              np.zeros((1, 7, 1, 1), np.float32), np.zeros((1, 7, 1, 1), np.float32), F32)
    o, _ = oracle.conv(one, np.ones((3, 1), np.float32), None, 1)
    want = np.array([float(v) / (1.0 + np.exp(-float(v))) for v in vals]).astype(np.float32)
    assert np.array_equal(o.x.ravel(), want)
    assert o.x.ravel()[3] == 0.0


def test_block_step_and_commit_with_conv():
    """With a width-1 identity convolution the conv variants are the plain calls; with a
    real one they are the plain calls on the convolved inputs, and the commit's conv state
    is the block's last W-1 raw rows."""
    rng = np.random.default_rng(24)
    b, T, H, P, N, G = 2, 12, 4, 3, 5, 2
    fwd = rand_seq(rng, b, T, H, P, N, G)
    rev = rand_seq(rng, b, T, H, P, N, G)
    A, D = rand_params(rng, H)
    h0 = 0.3 * rng.standard_normal((b, H, N, P))
    CH = H * P + 2 * G * N
    ident = (np.ones((CH, 1), np.float32), None, 0)
    y0 = oracle.block_step(h0, fwd, rev, A, D)[0]
    y1 = oracle.block_step_conv(h0, np.zeros((b, 0, CH), np.float32), fwd, rev, ident, ident, A, D)[0]
    assert np.array_equal(y0, y1)
    W = 4
    cf, cr = conv_weights(rng, CH, W), conv_weights(rng, CH, W)
    hist = rng.standard_normal((b, W - 1, CH)).astype(np.float32)
    y, _, _ = oracle.block_step_conv(h0, hist, fwd, rev, cf + (1,), cr + (1,), A, D)
    # the quadratic form on inputs convolved by the numpy reference
    def convolved(seq, wb, reverse, hs):
        v = conv_reference(raw_channels(seq), wb[0], wb[1], 1, reverse, hs)
        v = v.astype(np.float32)
        HP, GN = H * P, G * N
        return Seq(v[..., :HP].reshape(b, T, H, P).copy(), seq.dt, v[..., HP:HP + GN].reshape(b, T, G, N).copy(),
                   v[..., HP + GN:].reshape(b, T, G, N).copy(), F32)
    pf = convolved(fwd, cf, False, hist.astype(np.float64))
    pr = convolved(rev, cr, True, None)
    qf, _ = quad_forward(pf, A, D, h0, with_D=False)
    qr = quad_reverse(pr, A)
    expect = qf + qr + D[None, None, :, None] * dec(pf)[0]
    assert rel(y, expect) < 1e-6                      # float32 rounding of the convolved inputs
    hn, s_new, _ = oracle.commit_conv(h0, hist, fwd, cf + (1,), A, D)
    assert np.array_equal(s_new, raw_channels(fwd)[:, -(W - 1):].astype(np.float32))
    _, _, h_ref = oracle.scan(pf, A, D, chunk=T, h_init=h0)
    assert rel(hn, h_ref) < 1e-12


PLANTS = {
    "dropped dt on the input term": ("const double w = dt * val(in->B", "const double w = val(in->B"),
    "decay applied after the input": ("row[p] = alpha * row[p] + w * xv[p];",
                                      "row[p] = alpha * (row[p] + w * xv[p]);"),
    "reverse uses the forward dt": ("const double dt = val(rev->dt", "const double dt = val(fwd->dt"),
    "wrong group index": ("const int g = h / (H / G);\n    const int dty",
                          "const int g = h % G;\n    const int dty"),
    "D applied twice in the block step": ("(double)D[w] * val(fwd->x, dty, o);",
                                          "2.0 * (double)D[w] * val(fwd->x, dty, o);"),
    "reverse scan decays with the forward A": ("exp(dt * Ar[h])", "exp(dt * A[h])"),
    "reverse skip term on the forward input": ("(double)D_rev[w] * val(rev->x, dty, o)",
                                               "(double)D_rev[w] * val(fwd->x, dty, o)"),
    "C and B swapped in the forward output": (
        "acc += val(in->C, dty, (tok * G + g) * N + n) * S",
        "acc += val(in->B, dty, (tok * G + g) * N + n) * S"),
    "forward convolution taps reversed": ("const int64_t at = reverse ? t + width - 1 - k : t + k;",
                                          "const int64_t at = reverse ? t + width - 1 - k : t + width - 1 - k;"),
    "reverse convolution reads causally": ("const int64_t at = reverse ? t + width - 1 - k : t + k;",
                                           "const int64_t at = t + k;"),
    "conv state ignored": ("(!reverse && state_in) ?", "(0 && state_in) ?"),
    "conv state not advanced": ("u[len + k]);", "u[k]);"),
    "activation dropped": ("v = v / (1.0 + exp(-v));", "v = v * 1.0;"),
    "per-channel skip weight read per head": ("const int64_t w = skip_per_channel ? (int64_t)h * P + p : h;",
                                              "const int64_t w = skip_per_channel ? (int64_t)h * P : h;"),
    "full window drops the reverse parameters": ("zero, fwd, rev, A, D, A_rev, D_rev, y,",
                                                 "zero, fwd, rev, A, D, NULL, NULL, y,"),
}


def _planted_lib(tmp_path, name, old, new):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "bdssm_oracle.c")).read()
    assert src.count(old) >= 1, name
    path_c = tmp_path / "planted.c"
    path_c.write_text(src.replace(old, new))
    so = tmp_path / "planted.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(path_c), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_planted_mistake_is_caught(tmp_path, monkeypatch, name):
    old, new = PLANTS[name]
    so = _planted_lib(tmp_path, name, old, new)
    monkeypatch.setattr(oracle, "_LIB", so)
    monkeypatch.setattr(oracle, "_lib", None)
    failed = []
    for test in (test_golden_hand_worked, lambda: test_scan_matches_quadratic_form(F32, 2),
                 lambda: test_block_step_matches_quadratic_form(2),
                 test_block_step_separate_reverse_params,
                 lambda: test_conv_matches_shifted_slices(BF16, False),
                 lambda: test_conv_matches_shifted_slices(F32, True),
                 test_conv_identity_shift_and_flip, test_conv_state_chains_and_silu_values,
                 test_block_step_and_commit_with_conv, lambda: test_full_window_matches_quadratic_form(2),
                 test_block_step_per_channel_skip):
        try:
            test()
        except AssertionError:
            failed.append(test)
    monkeypatch.setattr(oracle, "_lib", None)
    assert failed, f"planted mistake '{name}' passed every pin"
